"""Repeated calls on the same inputs give bit-identical outputs (the measured workloads at full size), also when
calls run concurrently on two streams.

An engine that replays a step, or compares two runs of a request, needs the attention output to depend only on
the inputs: the kernels use no atomics in their arithmetic, the balanced decode's work division and the prefill
grid come from the lengths alone, and every reduction runs in a fixed order. Each workload below is called three
times (with other work on the cache pools in between for decode, whose step stores its new rows) and the outputs
are compared bit for bit; the workspace is refilled with NaN between calls, so no result may come from a
previous call's partials.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_111_amd as pa
from harness import DEV, DevStep, i32, to_dev
from workloads import make_config


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32).cpu().numpy() if t.dtype == torch.float32 else \
        t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["prefill_qwen3_8b", "chunked_qwen3_8b", "chunk256_qwen3_8b"])
def test_prefill_repeats_bit_for_bit(name):
    wl = make_config(name)
    st = wl.steps[-1]
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    ds = DevStep(st, wl.dtype)
    meta = pa.build_metadata_store(ds.num_cached, ds.num_new, ds.block_table, ds.total_q, ds.k, ds.v, kc, vc)
    mq, mk = int(st.num_new.max()), int((st.num_cached + st.num_new).max())
    need = pa.prefill_workspace_bytes(st.batch, wl.num_heads, wl.head_dim, mq, mk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
        out = pa.prefill_varlen(ds.q, kc, vc, meta["cu_seqlens_q"], meta["cu_seqlens_k"], ds.block_table, mq, mk,
                                wl.scale, out_dtype=torch.bfloat16, workspace=ws)
        torch.cuda.synchronize()
        outs.append(_bits(out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), f"{name}: outputs differ"


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["decode_qwen3_0p6b", "decode_qwen3_32b"])
def test_decode_step_repeats_bit_for_bit(name):
    wl = make_config(name)
    st = wl.steps[-1]
    kc, vc = to_dev(wl.k_cache, wl.dtype), to_dev(wl.v_cache, wl.dtype)
    ds = DevStep(st, wl.dtype)
    mbps = int(st.block_table.shape[1])
    ws = torch.empty(pa.decode_workspace_bytes(st.batch, wl.num_heads, wl.num_kv_heads, wl.head_dim, mbps,
                                               wl.block_size, 0), dtype=torch.uint8, device=DEV)
    outs = []
    for i in range(3):
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
        out = pa.decode_append(ds.q, ds.k, ds.v, kc, vc, ds.num_cached, ds.block_table, wl.scale,
                               out_dtype=torch.bfloat16, workspace=ws, fallback=False)
        torch.cuda.synchronize()
        outs.append(_bits(out))
        if i == 0:  # other work on the pools between calls: the step's own store again, then a plain decode
            ctx = i32(np.asarray(st.num_cached) + 1)
            pa.decode(ds.q, kc, vc, ctx, ds.block_table, wl.scale, workspace=ws)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), f"{name}: outputs differ"


@pytest.mark.gpu
def test_calls_on_two_streams_match_the_calls_alone():
    """The library keeps no state between calls but the caller's buffers: a decode step and a varlen prefill
    enqueued on two streams at once (each with its own pools and workspace) give the bits they give alone."""
    dec, pre = make_config("decode_qwen3_0p6b"), make_config("prefill_qwen3_8b")
    sd, sp = dec.steps[-1], pre.steps[-1]
    dkc, dvc = to_dev(dec.k_cache, dec.dtype), to_dev(dec.v_cache, dec.dtype)
    pkc, pvc = to_dev(pre.k_cache, pre.dtype), to_dev(pre.v_cache, pre.dtype)
    dds, pds = DevStep(sd, dec.dtype), DevStep(sp, pre.dtype)
    meta = pa.build_metadata_store(pds.num_cached, pds.num_new, pds.block_table, pds.total_q, pds.k, pds.v, pkc, pvc)
    mbps = int(sd.block_table.shape[1])
    dws = torch.empty(pa.decode_workspace_bytes(sd.batch, dec.num_heads, dec.num_kv_heads, dec.head_dim, mbps,
                                                dec.block_size, 0), dtype=torch.uint8, device=DEV)

    def run_decode(stream=None):
        return pa.decode_append(dds.q, dds.k, dds.v, dkc, dvc, dds.num_cached, dds.block_table, dec.scale,
                                workspace=dws, fallback=False, stream=stream)

    def run_prefill(stream=None):
        return pa.prefill_varlen(pds.q, pkc, pvc, meta["cu_seqlens_q"], meta["cu_seqlens_k"], pds.block_table,
                                 pds.max_q, pds.max_k, pre.scale, stream=stream)

    alone_d = _bits(run_decode())
    alone_p = _bits(run_prefill())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for _ in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            od = run_decode(stream=s1)
        with torch.cuda.stream(s2):
            op = run_prefill(stream=s2)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(od), alone_d), "decode on a second stream differs"
        assert np.array_equal(_bits(op), alone_p), "prefill on a second stream differs"
