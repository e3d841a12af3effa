"""The algorithmic work bench.py divides by (bytes for decode, flops for prefill), recounted independently.

Decode bytes count each KV row a call needs once: the test counts the distinct slots that the block tables
resolve the keys of every sequence to (sequences that share prefix blocks read those rows once). Prefill flops
count 4 * D * Hq per visible (query, key) pair: the test sums the visible keys row by row. The chunked
workload's pair count is the one its recipe fixes (2048 new rows after 30720 cached keys: 2048 * 30720 +
2048 * 2049 / 2 = 65 012 736).
"""

import numpy as np
import pytest

import bench
from workloads import make_config


def _distinct_rows(step, block_size):
    slots = []
    for s in range(step.batch):
        n = int(step.num_cached[s] + step.num_new[s])
        pos = np.arange(n)
        slots.append(step.block_table[s, pos // block_size].astype(np.int64) * block_size + pos % block_size)
    return np.unique(np.concatenate(slots)).size


@pytest.mark.parametrize("name", ["decode_qwen3_0p6b", "decode_qwen3_32b"])
def test_decode_bytes_count_each_needed_row_once(name):
    wl = make_config(name, fill=False)
    st = wl.steps[-1]
    work = bench.algorithmic_work(wl, st, 2)
    kv_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    assert work["kv_bytes"] == _distinct_rows(st, wl.block_size) * kv_tok
    B, T = st.batch, int(st.num_new.sum())
    qo = T * wl.num_heads * wl.head_dim * (wl.elem_bytes + 2)
    tables = sum(-(-int(c + n) // wl.block_size) for c, n in zip(st.num_cached, st.num_new))
    assert work["attn_bytes"] == work["kv_bytes"] + qo + 4 * tables + 4 * B
    if name == "decode_qwen3_32b":  # prefix sharing makes the distinct rows fewer than the sum of lengths
        assert work["kv_bytes"] < work["sum_k"] * kv_tok


@pytest.mark.parametrize("name", ["prefill_qwen3_8b", "chunked_qwen3_8b"])
def test_prefill_flops_count_visible_pairs(name):
    wl = make_config(name, fill=False)
    st = wl.steps[-1]
    pairs = 0
    for s in range(st.batch):
        q, c = int(st.num_new[s]), int(st.num_cached[s])
        pairs += int(np.sum(c + np.arange(q) + 1))  # row r sees keys 0 .. c + r
    work = bench.algorithmic_work(wl, st, 2)
    assert work["pairs"] == pairs
    assert work["flops"] == 4 * wl.head_dim * wl.num_heads * pairs
    if name == "chunked_qwen3_8b":
        assert pairs == 2048 * 30720 + 2048 * 2049 // 2 == 65_012_736


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // doubles x\n  return 2 * x;\n}\n/* block\n comment */\n"
    b = "// a new header line\nint f(int x) {  // twice x\n\n  return 2 * x;   \n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_text(a) == bench._code_text(b)
    assert bench._code_text(a) != bench._code_text(c)
