"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same seeded inputs.

Bit-exact for metadata (slots, prefix sums, lengths) and for the cache after store_kvcache; attention within
max-abs 2e-2 and relative RMS 5e-3 of the float64 oracle (bf16 inputs, float32 accumulation and output).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_111_amd as pa
from harness import DEV, MAX_ABS, REL_RMS, DevStep, assert_bf16_is_rounded_f32, assert_close, compare_metadata, \
    flat_rows, hip_step, i32, oracle_step, to_dev, to_host_bits
from workloads import build_decode, build_prefill, make_config

pytestmark = pytest.mark.gpu


def _run_and_check(wl, out_dtype=torch.float32, split_tokens=0, seqs=None, rows=None, check_pool=True,
                   fused_store=False, append=False):
    """Every step of the workload on both sides; returns the per-step (max_abs, rel_rms)."""
    kc_h, vc_h = wl.k_cache.copy(), wl.v_cache.copy()
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    errs = []
    for i, step in enumerate(wl.steps):
        print(f"[case] {wl.name} step {i} {step.kind} B={step.batch} T={step.num_tokens}", flush=True)
        ds = DevStep(step, wl.dtype)
        meta_d, out = hip_step(wl, ds, kc, vc, out_dtype=out_dtype, split_tokens=split_tokens,
                               fused_store=fused_store, append=append)
        out_f32 = None
        if out_dtype == torch.bfloat16:
            # the same step again with float32 output (its store rewrites the same rows with the same values)
            _, out_f32 = hip_step(wl, ds, kc, vc, out_dtype=torch.float32, split_tokens=split_tokens,
                                  fused_store=fused_store, append=append)
        torch.cuda.synchronize()
        meta_r, ref = oracle_step(wl, step, kc_h, vc_h, seqs=seqs, rows=rows)
        compare_metadata(meta_d, meta_r)
        if check_pool:
            assert np.array_equal(to_host_bits(kc), kc_h), "K cache differs after store"
            assert np.array_equal(to_host_bits(vc), vc_h), "V cache differs after store"
        frows = None if seqs is None else flat_rows(meta_r, seqs, rows)
        if out_f32 is not None:
            assert_close(out_f32, ref, frows, what=f"{wl.name} step {i} (float32 output)")
            assert_bf16_is_rounded_f32(out, out_f32, what=f"{wl.name} step {i}")
        err = assert_close(out, ref, frows, what=f"{wl.name} step {i}")
        print(f"[err] {wl.name} step {i}: max_abs {err[0]:.3e} rel_rms {err[1]:.3e}", flush=True)
        errs.append(err)
    return errs


# ------------------------------------------------------------------------------------------------ named configs


def test_tiny_config():
    _run_and_check(make_config("tiny"))


def test_decode_qwen3_0p6b_config():
    _run_and_check(make_config("decode_qwen3_0p6b"))


def test_prefill_qwen3_8b_config():
    _run_and_check(make_config("prefill_qwen3_8b"))


def test_chunked_qwen3_8b_config_all_rows():
    """All 2048 rows of the chunk (32 heads over 32768 keys) against the oracle, and the pool bit for bit."""
    _run_and_check(make_config("chunked_qwen3_8b"))


def test_chunk256_qwen3_8b_all_rows():
    """256 new rows over 32512 cached keys (eight key splits per workgroup and the merge pass), every row."""
    _run_and_check(make_config("chunk256_qwen3_8b"))


@pytest.fixture(scope="module")
def decode_32b():
    """The long-context decode workload with the oracle's answer for every sequence (computed once; the oracle's
    store writes the new rows into the host pools, which the device copies then start from: storing them again
    on the GPU writes the same bytes)."""
    wl = make_config("decode_qwen3_32b")
    meta_r, ref = oracle_step(wl, wl.steps[0], wl.k_cache, wl.v_cache)
    return wl, meta_r, ref


@pytest.mark.parametrize("append", [False, True])
def test_decode_qwen3_32b_config_all_sequences(decode_32b, append):
    """Full-size pool (offsets beyond 2^31 elements), all 256 sequences against the oracle; the store writes
    exactly the new rows (with append, the store is the decode call's own)."""
    wl, meta_r, ref = decode_32b
    step = wl.steps[0]
    print(f"[case] decode_qwen3_32b append={append} all sequences", flush=True)
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    row = wl.num_kv_heads * wl.head_dim
    slots = meta_r["slot_mapping"]
    idx = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    kc.view(-1, row)[idx] = 0  # the new rows start out different from what the step stores
    vc.view(-1, row)[idx] = 0
    kc0 = kc.clone()
    ds = DevStep(step, wl.dtype)
    meta_d, out = hip_step(wl, ds, kc, vc, append=append)
    torch.cuda.synchronize()
    compare_metadata(meta_d, meta_r)
    changed = torch.nonzero((kc.view(-1, row) != kc0.view(-1, row)).any(dim=1)).flatten().cpu().numpy()
    assert set(changed.tolist()) <= set(slots.tolist())
    assert np.array_equal(to_host_bits(kc.view(-1, row)[idx]), step.k.reshape(step.batch, row))
    assert np.array_equal(to_host_bits(vc.view(-1, row)[idx]), step.v.reshape(step.batch, row))
    del kc0
    err = assert_close(out, ref, what="decode_qwen3_32b")
    print(f"[err] decode_qwen3_32b append={append}: max_abs {err[0]:.3e} rel_rms {err[1]:.3e}", flush=True)


@pytest.mark.parametrize("split", [32, 256, 4096, 32768])
def test_decode_qwen3_32b_split_sizes(decode_32b, split):
    """Split-K with many, few and a single split per sequence gives the same answer within tolerance, on every
    sequence."""
    wl, _, ref = decode_32b
    step = wl.steps[0]
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    ds = DevStep(step, wl.dtype)
    print(f"[case] decode_qwen3_32b split {split}", flush=True)
    _, out = hip_step(wl, ds, kc, vc, split_tokens=split)
    torch.cuda.synchronize()
    assert_close(out, ref, what=f"split {split}")


# ------------------------------------------------------------------------------------------------ small shapes

def _short_prompts(seed: int, n: int):
    """n prompts of 1..199 tokens, about half of them after a cached 16-token block (when longer than it)."""
    rng = np.random.default_rng(seed)
    k_lens = rng.integers(1, 200, n)
    cached = np.minimum(rng.integers(0, 2, n) * 16, k_lens - 1)
    return [int(x) for x in k_lens], [int(x) for x in cached]


PREFILL_CASES = [
    # Hq, Hkv, D, bs, dtype, k_lens, cached
    (32, 8, 128, 256, "bf16", [300, 129, 1000, 17], [256, 0, 512, 0]),
    (8, 8, 128, 16, "bf16", [77, 200, 33, 1], [10, 150, 0, 0]),
    (16, 1, 128, 32, "bf16", [260, 5, 64], [3, 0, 63]),
    (12, 4, 128, 24, "bf16", [100, 61, 130], [50, 0, 129]),
    (4, 2, 64, 16, "bf16", [40, 17], [8, 0]),
    (8, 2, 128, 16, "f32", [70, 33], [20, 0]),
    (4, 4, 16, 4, "f32", [9, 13], [0, 5]),
    (32, 8, 128, 256, "bf16", [2048], [0]),
    # two query heads per KV head with a block size that is not a power of two (tiles gathered key by key);
    # 64-key blocks with one-key sequences and a chunk that starts inside a block
    (8, 4, 128, 24, "bf16", [100, 61, 130], [50, 0, 129]),
    (16, 8, 128, 64, "bf16", [500, 64, 65, 1], [436, 0, 1, 0]),
    # block size 1 (every key its own block)
    (8, 2, 128, 1, "bf16", [17, 5], [3, 0]),
    # 512-key blocks; 16 query heads per KV head
    (16, 1, 128, 512, "bf16", [1100, 513, 40], [512, 0, 39]),
    # 64 sequences (the most the kernel numbers by existing row blocks) and 70 (numbered over the whole grid),
    # short mixed prompts, some after a cached prefix
    (8, 2, 128, 16, "bf16", *_short_prompts(11, 64)),
    (8, 2, 128, 16, "bf16", *_short_prompts(13, 70)),
    # a prompt of more than 63 x 128 rows (numbered over the whole grid as well) after a cached prefix
    (8, 2, 128, 256, "bf16", [8500], [300]),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_small(case):
    Hq, Hkv, D, bs, dt, kl, cached = PREFILL_CASES[case]
    wl = build_prefill(f"prefill_small_{case}", 200 + case, Hq, Hkv, D, bs, dt, kl, cached,
                       num_blocks=sum(-(-n // bs) for n in kl) + 3)
    _run_and_check(wl)


DECODE_CASES = [
    # Hq, Hkv, D, bs, dtype, ctx, split
    (16, 8, 128, 256, "bf16", [1, 255, 256, 257, 4096, 1000], 0),
    (16, 8, 128, 256, "bf16", [1, 255, 256, 257, 4096, 1000], 32),
    (64, 8, 128, 256, "bf16", [33, 700, 2049], 256),
    (16, 1, 128, 16, "bf16", [50, 17, 300], 64),
    (8, 2, 128, 24, "bf16", [100, 49, 1], 96),
    (32, 1, 128, 16, "bf16", [40, 90], 0),
    (8, 2, 128, 16, "f32", [70, 33], 0),
    (4, 2, 64, 16, "bf16", [70, 33], 0),
    # balanced decode (split_tokens = 0, D = 128, block size a multiple of 32): G = 16 with 32-key blocks; many
    # short mixed lengths; one long sequence whose pairs are cut across more than 64 worker slices
    (16, 1, 128, 32, "bf16", [1, 31, 32, 33, 5000], 0),
    (32, 8, 128, 64, "bf16", [int(x) for x in np.random.default_rng(7).integers(1, 600, 300)], 0),
    (8, 8, 128, 256, "bf16", [20000], 0),
    # a block size that is a multiple of 32 but not a power of two (balanced decode, divided block index);
    # new keys at a block's first and last slot
    (8, 2, 128, 96, "bf16", [1, 96, 97, 500, 192, 191], 0),
    # 3 KV heads: the balanced decode's groups of Hkv workers do not divide its worker count
    (12, 3, 128, 64, "bf16", [5, 700, 64, 65, 1000, 3000], 0),
    # 64 KV heads, one query head each (groups of 64 workers); 512-key blocks
    (64, 64, 128, 32, "bf16", [100, 3000, 33], 0),
    (16, 8, 128, 512, "bf16", [1, 511, 512, 513, 2600], 0),
    # block size 1; 32 query heads per KV head (beyond the MFMA kernels' 16: the generic kernel)
    (8, 2, 128, 1, "bf16", [17, 1, 40], 0),
    (32, 1, 128, 16, "bf16", [50, 300], 0),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_small(case):
    Hq, Hkv, D, bs, dt, ctx, split = DECODE_CASES[case]
    wl = build_decode(f"decode_small_{case}", 300 + case, Hq, Hkv, D, bs, dt, ctx,
                      num_blocks=sum(-(-n // bs) for n in ctx) + 2)
    _run_and_check(wl, split_tokens=split)


# few query tiles over long keys: the prefill kernel splits each workgroup's key tiles (fewer workgroups than the
# chip runs at once) and a merge pass combines the splits' partials. Chunks of 200 rows and of one row over
# thousands of cached keys; a mixed batch where some rows see no key in a split (their split partial is empty);
# 16-key blocks (tiles gathered key by key); sequences without new tokens
PREFILL_SPLIT_CASES = [
    # Hq, Hkv, D, bs, dtype, k_lens, cached, out_dtype
    (32, 8, 128, 256, "bf16", [8392], [8192], "f32"),
    (32, 8, 128, 256, "bf16", [5001], [5000], "f32"),
    (8, 2, 128, 256, "bf16", [3000, 4100, 1500], [2900, 3800, 0], "f32"),
    (16, 4, 128, 16, "bf16", [2100], [2000], "bf16"),
    (16, 8, 128, 256, "bf16", [5005, 9000, 70], [5000, 9000, 0], "f32"),
]


@pytest.mark.parametrize("case", range(len(PREFILL_SPLIT_CASES)))
def test_prefill_key_splits(case):
    Hq, Hkv, D, bs, dt, kl, cached, odt = PREFILL_SPLIT_CASES[case]
    q_lens = [k - c for k, c in zip(kl, cached)]
    need = pa.prefill_workspace_bytes(len(kl), Hq, D, max(q_lens), max(kl))
    assert need > 0, "the case must take the split path"
    wl = build_prefill(f"prefill_split_{case}", 700 + case, Hq, Hkv, D, bs, dt, kl, cached,
                       num_blocks=sum(-(-n // bs) for n in kl) + 3, allow_empty=0 in q_lens)
    _run_and_check(wl, out_dtype=torch.bfloat16 if odt == "bf16" else torch.float32)


@pytest.mark.parametrize("bs", [16, 256])
def test_prefill_with_sequences_without_new_tokens(bs):
    """Sequences with no new token in a prefill batch compute nothing and leave the others unchanged."""
    kl, cached = ([40, 33, 70, 16], [40, 5, 70, 0]) if bs == 16 else ([300, 257, 512], [300, 0, 512])
    wl = build_prefill(f"prefill_empty_{bs}", 610 + bs, 8, 2, 128, bs, "bf16", kl, cached,
                       num_blocks=sum(-(-n // bs) for n in kl) + 2, allow_empty=True)
    _run_and_check(wl)


def test_decode_batch_beyond_the_balanced_limit():
    """5000 sequences (more than the 4096 whose prefix sums the balanced decode and the metadata build keep in
    LDS): with slots and lengths from the host, pa_store_kvcache and pa_decode (its fixed-split kernels) match
    the oracle; pa_decode_append refuses the batch before launching, as its fallback's metadata build does."""
    ctx = [int(x) for x in np.random.default_rng(12).integers(1, 90, 5000)]
    wl = build_decode("decode_5000", 621, 8, 2, 128, 32, "bf16", ctx, num_blocks=sum(-(-n // 32) for n in ctx) + 2)
    step = wl.steps[0]
    kc_h, vc_h = wl.k_cache.copy(), wl.v_cache.copy()
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    ds = DevStep(step, wl.dtype)
    print("[case] decode_5000", flush=True)
    meta_r, ref = oracle_step(wl, step, kc_h, vc_h)
    pa.store_kvcache(ds.k, ds.v, kc, vc, i32(meta_r["slot_mapping"]))
    out = pa.decode(ds.q, kc, vc, i32(meta_r["context_lens"]), ds.block_table, wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(kc), kc_h) and np.array_equal(to_host_bits(vc), vc_h)
    assert_close(out, ref, what="decode 5000")
    kc0 = kc.clone()
    with pytest.raises(pa.PAError, match="UNSUPPORTED"):
        pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale, fallback=False)
    with pytest.raises(pa.PAError, match="SHAPE"):
        pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc0)


def test_decode_largest_batch():
    """4096 sequences (the largest batch of the balanced decode's prefix sums) of 1..64 keys."""
    ctx = [int(x) for x in np.random.default_rng(11).integers(1, 65, 4096)]
    wl = build_decode("decode_4096", 620, 8, 2, 128, 32, "bf16", ctx, num_blocks=sum(-(-n // 32) for n in ctx) + 2)
    _run_and_check(wl)


# the decode step with the new K/V given (pa_decode_append: store inside the balanced decode's pass) on every
# decode shape it takes: 1..20000 keys, block sizes 32 to 256 (96 among them), G = 2 to 16, 300 and 4096
# sequences, the Qwen3-0.6B workload's steps; the caches must match the oracle's bit for bit after each step
APPEND_CASES = [0, 8, 9, 10, 11, 12, 13, 14]


@pytest.mark.parametrize("case", APPEND_CASES)
def test_decode_append(case):
    Hq, Hkv, D, bs, dt, ctx, _ = DECODE_CASES[case]
    wl = build_decode(f"append_decode_{case}", 300 + case, Hq, Hkv, D, bs, dt, ctx,
                      num_blocks=sum(-(-n // bs) for n in ctx) + 2)
    _run_and_check(wl, append=True)


def test_decode_append_qwen3_0p6b_config_and_largest_batch():
    _run_and_check(make_config("decode_qwen3_0p6b"), append=True)
    ctx = [int(x) for x in np.random.default_rng(11).integers(1, 65, 4096)]
    wl = build_decode("append_decode_4096", 620, 8, 2, 128, 32, "bf16", ctx,
                      num_blocks=sum(-(-n // 32) for n in ctx) + 2)
    _run_and_check(wl, append=True, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("case", [3, 6, 16])
def test_decode_append_falls_back_on_other_shapes(case):
    """Block size 16, float32, 32 query heads per KV head: the binding stores and decodes in separate calls."""
    Hq, Hkv, D, bs, dt, ctx, _ = DECODE_CASES[case]
    wl = build_decode(f"append_fallback_{case}", 300 + case, Hq, Hkv, D, bs, dt, ctx,
                      num_blocks=sum(-(-n // bs) for n in ctx) + 2)
    ds = DevStep(wl.steps[0], wl.dtype)
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale, fallback=False)
    kc_h, vc_h = wl.k_cache.copy(), wl.v_cache.copy()
    for i, step in enumerate(wl.steps):
        ds = DevStep(step, wl.dtype)
        out = pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale)
        torch.cuda.synchronize()
        _, ref = oracle_step(wl, step, kc_h, vc_h)
        assert np.array_equal(to_host_bits(kc), kc_h) and np.array_equal(to_host_bits(vc), vc_h)
        assert_close(out, ref, what=f"fallback {case} step {i}")


# metadata and store in one launch (pa_build_metadata_store) on shapes of the cases above: bf16 and f32 rows of
# 64 to 4096 bytes, block sizes 1 to 256, sequences without new tokens, 300 and 4096 sequences
FUSED_STORE_CASES = [("prefill", 0), ("prefill", 4), ("prefill", 5), ("prefill", 6), ("prefill", 10),
                     ("decode", 0), ("decode", 9), ("decode", 11), ("decode", 15)]


@pytest.mark.parametrize("case", FUSED_STORE_CASES)
def test_fused_metadata_store(case):
    kind, i = case
    if kind == "prefill":
        Hq, Hkv, D, bs, dt, kl, cached = PREFILL_CASES[i]
        wl = build_prefill(f"fused_prefill_{i}", 200 + i, Hq, Hkv, D, bs, dt, kl, cached,
                           num_blocks=sum(-(-n // bs) for n in kl) + 3)
    else:
        Hq, Hkv, D, bs, dt, ctx, _ = DECODE_CASES[i]
        wl = build_decode(f"fused_decode_{i}", 300 + i, Hq, Hkv, D, bs, dt, ctx,
                          num_blocks=sum(-(-n // bs) for n in ctx) + 2)
    _run_and_check(wl, fused_store=True)


def test_fused_metadata_store_empty_sequences_and_large_batch():
    kl, cached = [40, 33, 70, 16], [40, 5, 70, 0]
    wl = build_prefill("fused_prefill_empty", 626, 8, 2, 128, 16, "bf16", kl, cached,
                       num_blocks=sum(-(-n // 16) for n in kl) + 2, allow_empty=True)
    _run_and_check(wl, fused_store=True)
    ctx = [int(x) for x in np.random.default_rng(11).integers(1, 65, 4096)]
    wl = build_decode("fused_decode_4096", 620, 8, 2, 128, 32, "bf16", ctx,
                      num_blocks=sum(-(-n // 32) for n in ctx) + 2)
    _run_and_check(wl, fused_store=True)


@pytest.mark.parametrize("hkv, stride_pad", [(32, 0), (8, 1)])
def test_fused_metadata_store_wide_and_unaligned_rows(hkv, stride_pad):
    """Rows of 8 KiB (past what the kernel keeps in registers) and rows whose token stride is odd (2-byte copies),
    as views of a fused projection output; metadata and cache bit-exact against the oracle."""
    D, bs, hq = 128, 16, 8
    rng = np.random.default_rng(40 + hkv)
    cached = np.array([3, 0, 17, 40], np.int64)
    new = np.array([5, 12, 1, 0], np.int64)
    nbk = [-(-int(c + n) // bs) for c, n in zip(cached, new)]
    nb = sum(nbk) + 4
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((4, max(nbk)), -1, np.int32)
    at = 0
    for s in range(4):
        table[s, :nbk[s]] = perm[at:at + nbk[s]]
        at += nbk[s]
    T = int(new.sum())
    width = (hq + 2 * hkv) * D + stride_pad
    qkv = torch.from_numpy(rng.standard_normal((T, width)).astype(np.float32)).to(DEV).bfloat16()
    k = qkv[:, hq * D:(hq + hkv) * D].view(T, hkv, D)
    v = qkv[:, (hq + hkv) * D:(hq + 2 * hkv) * D].view(T, hkv, D)
    kc_h = rng.standard_normal((nb, bs, hkv, D)).astype(np.float32)
    kc = torch.from_numpy(kc_h).to(DEV).bfloat16()
    vc = kc.clone()
    ref_k, ref_v = to_host_bits(kc), to_host_bits(vc)
    meta = pa.build_metadata_store(i32(cached), i32(new), i32(table), T, k, v, kc, vc)
    ref = oracle.build_metadata(table, cached, new, bs)
    compare_metadata(meta, ref)
    oracle.store_kvcache(ref_k, ref_v, to_host_bits(k.contiguous()), to_host_bits(v.contiguous()),
                         ref["slot_mapping"])
    assert np.array_equal(to_host_bits(kc), ref_k) and np.array_equal(to_host_bits(vc), ref_v)


def test_bf16_output():
    wl = build_prefill("bf16_out", 400, 32, 8, 128, 256, "bf16", [300, 700], [256, 0])
    _run_and_check(wl, out_dtype=torch.bfloat16)
    wl = build_decode("bf16_out_d", 401, 16, 8, 128, 256, "bf16", [300, 3000])
    _run_and_check(wl, out_dtype=torch.bfloat16, split_tokens=256)


# ------------------------------------------------------------------------------------------------ properties


def _relabel(wl, perm):
    kc = np.empty_like(wl.k_cache)
    vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache
    vc[perm] = wl.v_cache
    st = wl.steps[0]
    bt = np.where(st.block_table >= 0, perm[np.maximum(st.block_table, 0)], -1).astype(np.int32)
    return kc, vc, type(st)(st.kind, bt, st.num_cached, st.num_new, st.q, st.k, st.v)


@pytest.mark.parametrize("kind", ["prefill", "prefill_split", "decode"])
def test_physical_relabelling_is_bit_identical(kind):
    if kind == "prefill":
        wl = build_prefill("perm_p", 500, 32, 8, 128, 64, "bf16", [300, 129, 500], [64, 0, 128], num_blocks=20)
    elif kind == "prefill_split":  # key splits + merge (one 100-row chunk over 4000 keys)
        wl = build_prefill("perm_ps", 502, 32, 8, 128, 64, "bf16", [4100], [4000], num_blocks=70)
        assert pa.prefill_workspace_bytes(1, 32, 128, 100, 4100) > 0
    else:
        wl = build_decode("perm_d", 501, 64, 8, 128, 64, "bf16", [300, 129, 1500], num_blocks=40)
    perm = np.random.default_rng(3).permutation(wl.num_blocks)
    kc2, vc2, st2 = _relabel(wl, perm)
    outs = []
    for kch, vch, st in ((wl.k_cache, wl.v_cache, wl.steps[0]), (kc2, vc2, st2)):
        kc, vc = to_dev(kch, wl.dtype), to_dev(vch, wl.dtype)
        _, out = hip_step(wl, DevStep(st, wl.dtype), kc, vc, split_tokens=128)
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("kind", ["prefill", "prefill_split", "decode"])
def test_nan_in_unreferenced_slots_does_not_reach_output(kind):
    if kind == "prefill":
        wl = build_prefill("nan_p", 510, 32, 8, 128, 256, "bf16", [300, 77], [256, 0], num_blocks=6)
    elif kind == "prefill_split":  # the key ranges of the splits end inside blocks whose tails hold NaN
        wl = build_prefill("nan_ps", 512, 32, 8, 128, 256, "bf16", [3000, 77], [2950, 0], num_blocks=16)
        assert pa.prefill_workspace_bytes(2, 32, 128, 77, 3000) > 0
    else:
        wl = build_decode("nan_d", 511, 16, 8, 128, 256, "bf16", [300, 77, 513], num_blocks=8)
    st = wl.steps[0]
    k_len = st.num_cached + st.num_new
    keep = np.zeros(wl.num_blocks * wl.block_size, bool)
    for s in range(st.batch):
        ids = st.block_table[s][:oracle.num_blocks(int(k_len[s]), wl.block_size)]
        keep[oracle.get_slots(ids, wl.block_size, int(k_len[s]))] = True
    outs = []
    for poison in (False, True):
        kch, vch = wl.k_cache.copy(), wl.v_cache.copy()
        if poison:
            kch.reshape(-1, wl.num_kv_heads, wl.head_dim)[~keep] = 0x7FC0  # bf16 quiet NaN
            vch.reshape(-1, wl.num_kv_heads, wl.head_dim)[~keep] = 0x7FC0
        kc, vc = to_dev(kch, wl.dtype), to_dev(vch, wl.dtype)
        _, out = hip_step(wl, DevStep(st, wl.dtype), kc, vc, split_tokens=64)
        outs.append(out.cpu())
    assert torch.isfinite(outs[1]).all()
    assert torch.equal(outs[0], outs[1])


def test_store_slot_102_changes_exactly_one_row():
    """The worked slot example on the device: one token stored at slot 25*4+2 of a bs=4 pool."""
    nb, bs, Hkv, D = 32, 4, 2, 16
    rng = np.random.default_rng(9)
    kc_h = rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    kc, vc = to_dev(kc_h, "f32"), to_dev(kc_h, "f32")
    k = torch.from_numpy(rng.standard_normal((3, Hkv, D)).astype(np.float32)).to(DEV)
    pa.store_kvcache(k, k, kc, vc, i32([-1, oracle.slot_of(25, 4, 2), -1]))
    got = to_host_bits(kc)
    diff = np.flatnonzero((got != kc_h).reshape(-1))
    row = Hkv * D
    assert diff.min() >= 102 * row and diff.max() < 103 * row
    assert np.array_equal(got[25, 2], k[1].cpu().numpy())


def test_store_from_strided_fused_qkv():
    """k and v as views of a fused [T, (Hq + 2 Hkv) * D] projection output (token stride > row)."""
    Hq, Hkv, D, bs, nb, T = 32, 8, 128, 256, 8, 300
    rng = np.random.default_rng(10)
    qkv = torch.from_numpy(rng.standard_normal((T, (Hq + 2 * Hkv) * D)).astype(np.float32)).to(DEV).bfloat16()
    k = qkv[:, Hq * D:(Hq + Hkv) * D].view(T, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].view(T, Hkv, D)
    kc = torch.zeros((nb, bs, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    pa.store_kvcache(k, v, kc, vc, i32(slots))
    kh, vh = to_host_bits(kc).reshape(nb * bs, -1), to_host_bits(vc).reshape(nb * bs, -1)
    ref_k = np.zeros_like(kh)
    ref_v = np.zeros_like(vh)
    oracle.store_kvcache(ref_k.reshape(nb, bs, Hkv, D), ref_v.reshape(nb, bs, Hkv, D),
                         to_host_bits(k.contiguous()), to_host_bits(v.contiguous()), slots)
    assert np.array_equal(kh, ref_k) and np.array_equal(vh, ref_v)


def test_metadata_prepare_prefill_example(golden):
    g = golden["prepare_prefill"]
    table = i32([[7], [3]])
    meta = pa.build_metadata(i32([0, 0]), i32([3, 2]), table, 5, 16, g["block_size"])
    assert meta["positions"].cpu().tolist() == g["positions"]
    assert meta["cu_seqlens_q"].cpu().tolist() == g["cu_seqlens_q"]
    assert meta["slot_mapping"].cpu().tolist() == g["slot_mapping"]


def test_metadata_chunked_counters_example(golden):
    g = golden["chunked_counters"]
    table = i32([g["block_table"]])
    full = oracle.get_slots(g["block_table"], g["block_size"], g["prompt"])
    for ch in g["chunks"]:
        meta = pa.build_metadata(i32([ch["num_cached"]]), i32([ch["num_scheduled"]]), table, ch["num_scheduled"],
                                 16, g["block_size"])
        assert meta["context_lens"].cpu().tolist() == [ch["cached_after"]]
        assert meta["slot_mapping"].cpu().tolist() == full[ch["num_cached"]:ch["cached_after"]]


def test_metadata_large_batch_bit_exact():
    rng = np.random.default_rng(11)
    B, bs = 3000, 16
    cached = rng.integers(0, 200, B)
    new = rng.integers(0, 40, B)
    nbk = [-(-(int(c) + int(n)) // bs) for c, n in zip(cached, new)]
    perm = rng.permutation(sum(nbk) + 5).astype(np.int32)
    width = max(nbk)
    table = np.full((B, width), -1, np.int32)
    at = 0
    for s in range(B):
        table[s, :nbk[s]] = perm[at:at + nbk[s]]
        at += nbk[s]
    ref = oracle.build_metadata(table, cached, new, bs)
    meta = pa.build_metadata(i32(cached), i32(new), i32(table), int(new.sum()), len(perm), bs)
    compare_metadata(meta, ref)


# ------------------------------------------------------------------------------------------------ PV precision


def _f16_toward_zero(x: np.ndarray) -> np.ndarray:
    """float32 -> the fp16 value rounding toward zero, as float32: finite magnitudes above 65504 become +-65504,
    magnitudes below 2^-14 fp16 subnormals (truncated) or zero. Written from the IEEE half format with NumPy's
    float16 (round to nearest), stepped one ulp toward zero where that rounded away from zero."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    away = np.abs(h.astype(np.float32)) > np.abs(x)
    h = np.where(away, np.nextafter(h, np.float16(0)), h)
    h = np.where(np.abs(x) > 65504, np.sign(x).astype(np.float16) * np.float16(65504), h)
    return h.astype(np.float32)


@pytest.mark.parametrize("mode", ["large", "tiny"])
def test_prefill_pv_range_rule(mode):
    """The bf16 head_dim-128 prefill runs its PV product in fp16 with V converted toward zero (the rule stated in
    pa.h for pa_prefill_varlen). V holding +-1e5 entries (beyond fp16's 65504) or only magnitudes near 1e-6 (fp16
    subnormals): the output follows the oracle run on the converted V, and differs from the oracle on the raw V
    by far more than that, so the rule is what the kernel computes."""
    wl = build_prefill("pv_range", 731, 8, 2, 128, 64, "bf16", [320], [128], num_blocks=12)
    st = wl.steps[0]
    rng = np.random.default_rng(5)

    def f32(bits):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)

    def bits(x):
        return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
            np.uint16)

    vp, vn = f32(wl.v_cache), f32(st.v)
    if mode == "large":
        for a in (vp, vn):
            hit = rng.random(a.shape) < 0.05
            a[hit] = np.sign(rng.standard_normal(int(hit.sum()))) * 1e5
    else:
        vp *= 1e-6
        vn *= 1e-6
    wl.v_cache[...] = bits(vp)
    st.v[...] = bits(vn)
    kc_h, vc_h = wl.k_cache.copy(), wl.v_cache.copy()
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    print(f"[case] pv_range {mode}", flush=True)
    meta_d, out = hip_step(wl, DevStep(st, wl.dtype), kc, vc)
    torch.cuda.synchronize()
    meta_r, plain = oracle_step(wl, st, kc_h, vc_h)
    compare_metadata(meta_d, meta_r)
    rule = oracle.prefill_varlen(f32(st.q), f32(kc_h), _f16_toward_zero(f32(vc_h)), meta_r["cu_seqlens_q"],
                                 meta_r["cu_seqlens_k"], st.block_table, wl.scale, "f32")
    got = out.float().cpu().numpy().astype(np.float64)

    def rel(a, b):
        return float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b * b)))

    r_rule, r_plain = rel(got, rule), rel(got, plain)
    print(f"[err] pv_range {mode}: rel_rms vs rule {r_rule:.2e}, vs raw V {r_plain:.2e}", flush=True)
    assert r_rule <= REL_RMS, f"{mode}: output is not the stated rule's ({r_rule:.3g})"
    assert r_plain > 5 * max(r_rule, 1e-3), f"{mode}: the rule is not observable ({r_plain:.3g} vs {r_rule:.3g})"
    # elementwise: the fp16 weights (relative 2^-11 each) bound the error by 2^-11 of the largest |V'| reached
    bound = MAX_ABS + 2.0 ** -11 * float(np.max(np.abs(_f16_toward_zero(f32(vc_h)))))
    assert np.max(np.abs(got - rule)) <= bound
