"""pa_decode_append_noalloc (the decode step with its partials in the library's own device scratch) against
pa_decode_append (the same step with a caller workspace), through the C ABI: two calls in a row on one GPU, the
second with a smaller batch, each bit for bit equal to the workspace call on a copy of the caches and within the
attention tolerance of the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_111_amd as pa
from harness import DEV, assert_close

HQ, HKV, D, BS = 16, 8, 128, 256


def _bf16(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.gpu
def test_noalloc_decode_append_matches_the_workspace_call_on_two_calls():
    rng = np.random.default_rng(4242)
    mbps = 16
    nb = 64 * mbps + 8
    table = rng.permutation(nb).astype(np.int32)[: 64 * mbps].reshape(64, mbps)
    pool_k, pool_v = _bf16(rng, (nb, BS, HKV, D)), _bf16(rng, (nb, BS, HKV, D))
    kc_n, vc_n = pool_k.to(DEV), pool_v.to(DEV)  # the no-allocation call's caches
    kc_w, vc_w = kc_n.clone(), vc_n.clone()      # the workspace call's caches
    kc_h, vc_h = _bits(pool_k).copy(), _bits(pool_v).copy()  # the oracle's
    scale = 1.0 / np.sqrt(D)
    ws = torch.empty(pa.decode_workspace_bytes(64, HQ, HKV, D, mbps, BS, 0), dtype=torch.uint8, device=DEV)
    for call, batch in enumerate((64, 9)):  # the second call is smaller
        print(f"[case] noalloc call {call} batch {batch}", flush=True)
        cached = rng.integers(0, mbps * BS, size=batch).astype(np.int32)
        q, k, v = _bf16(rng, (batch, HQ, D)), _bf16(rng, (batch, HKV, D)), _bf16(rng, (batch, HKV, D))
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        nc = torch.from_numpy(cached).to(DEV)
        bt = torch.from_numpy(np.ascontiguousarray(table[:batch])).to(DEV)
        out_n = torch.empty((batch, HQ, D), dtype=torch.float32, device=DEV)
        out_w = torch.empty_like(out_n)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        pa.decode_append_noalloc(qd, kd, vd, kc_n, vc_n, nc, bt, scale, out=out_n)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        pa.decode_append(qd, kd, vd, kc_w, vc_w, nc, bt, scale, out=out_w, workspace=ws, fallback=False)
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_w), f"call {call}: output differs from pa_decode_append"
        assert torch.equal(kc_n, kc_w) and torch.equal(vc_n, vc_w), f"call {call}: caches differ"
        slots = (table[np.arange(batch), cached // BS].astype(np.int64) * BS + cached % BS).astype(np.int32)
        oracle.store_kvcache(kc_h, vc_h, _bits(k), _bits(v), slots)
        ref = oracle.decode(_bits(q), kc_h, vc_h, cached + 1, table[:batch], scale, "bf16")
        assert np.array_equal(_bits(kc_n.cpu()), kc_h) and np.array_equal(_bits(vc_n.cpu()), vc_h)
        err = assert_close(out_n, ref, what=f"noalloc call {call}")
        print(f"[err] noalloc call {call}: max_abs {err[0]:.2e} rel_rms {err[1]:.2e}", flush=True)


@pytest.mark.gpu
def test_noalloc_refuses_what_the_workspace_call_refuses():
    """A shape the balanced decode does not take (block size 16) is refused before anything runs."""
    rng = np.random.default_rng(7)
    kc = _bf16(rng, (8, 16, HKV, D)).to(DEV)
    vc = kc.clone()
    q = _bf16(rng, (2, HQ, D)).to(DEV)
    k = _bf16(rng, (2, HKV, D)).to(DEV)
    nc = torch.tensor([3, 5], dtype=torch.int32, device=DEV)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=DEV)
    out = torch.empty((2, HQ, D), dtype=torch.float32, device=DEV)
    with pytest.raises(pa.PAError, match="UNSUPPORTED"):
        pa.decode_append_noalloc(q, k, k, kc, vc, nc, bt, 0.1, out=out)
