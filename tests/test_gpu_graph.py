"""Store + decode captured once in a HIP graph and replayed with new inputs.

Every call of the library only enqueues work on the caller's stream, with grids computed from host scalars
(batch, table width, block size), no allocation, no memset and no host read of device data, so one capture
serves later decode steps of the same batch size whose lengths, slots, queries and new K/V change in device
memory (the engine captures only its decode step and replays it with new data copied into fixed tensors,
"一个 prompt 的一生：nano-vllm 从起服务到吐出 token" §2.2.4).
Each replay is checked bit for bit against the same calls run eagerly on a second copy of the cache pool, with
eager work and synchronisations between replays; the decode-step replays are also checked against the oracle
(the first and the last replay of each capture, over host pools that received every replay's stores), up to
batch 512, the largest batch the engine captures ("一个 prompt 的一生" §3.3.2).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_111_amd as pa
from harness import DEV, assert_close

HQ, HKV, D, BS = 16, 8, 128, 256


def _bf16(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    return x.to(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


class HostMirror:
    """The oracle's side of a captured decode step: host pools that receive every replay's stores through the
    oracle's store_kvcache, and the oracle's decode of a replay's step over them."""

    def __init__(self, pool_k: torch.Tensor, pool_v: torch.Tensor, table: np.ndarray):
        self.kc, self.vc = _bits(pool_k).copy(), _bits(pool_v).copy()
        self.table = table

    def store(self, k_new: torch.Tensor, v_new: torch.Tensor, slots: np.ndarray) -> None:
        oracle.store_kvcache(self.kc, self.vc, _bits(k_new), _bits(v_new), slots)

    def check(self, out: torch.Tensor, q: torch.Tensor, ctx: np.ndarray, kc_dev: torch.Tensor, what: str) -> None:
        ref = oracle.decode(_bits(q), self.kc, self.vc, ctx, self.table, 1.0 / np.sqrt(D), "bf16")
        assert np.array_equal(_bits(kc_dev.cpu()), self.kc), f"{what}: K pool differs from the oracle's"
        assert_close(out, ref, what=what)


def _slots(table: np.ndarray, pos: np.ndarray) -> np.ndarray:
    return (table[np.arange(len(pos)), pos // BS].astype(np.int64) * BS + pos % BS).astype(np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("batch,split", [(1, 0), (4, 0), (16, 0), (8, 256), (512, 0)])
def test_graph_store_decode_replays(batch, split):
    rng = np.random.default_rng(900 + batch + split)
    mbps = 4 if batch > 64 else 8              # up to 1024 (2048) keys per sequence
    nb = batch * mbps + 4
    perm = rng.permutation(nb).astype(np.int32)
    table = perm[: batch * mbps].reshape(batch, mbps)
    pool_k = _bf16(rng, (nb, BS, HKV, D))
    pool_v = _bf16(rng, (nb, BS, HKV, D))
    host = HostMirror(pool_k, pool_v, table)
    kc_g, vc_g = pool_k.to(DEV), pool_v.to(DEV)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()

    # static device buffers the graph reads
    q = torch.empty((batch, HQ, D), dtype=torch.bfloat16, device=DEV)
    k_new = torch.empty((batch, HKV, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    slots = torch.empty(batch, dtype=torch.int32, device=DEV)
    ctx = torch.empty(batch, dtype=torch.int32, device=DEV)
    bt = torch.from_numpy(table).to(DEV)
    out_g = torch.empty((batch, HQ, D), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    need = pa.decode_workspace_bytes(batch, HQ, HKV, D, mbps, BS, split)
    ws_g = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws_g)
    scale = 1.0 / np.sqrt(D)
    cur = {}

    def draw():
        lens = rng.integers(1, mbps * BS + 1, size=batch).astype(np.int32)
        sl = _slots(table, lens - 1)
        cur.update(q=_bf16(rng, (batch, HQ, D)), k=_bf16(rng, (batch, HKV, D)), v=_bf16(rng, (batch, HKV, D)),
                   lens=lens, slots=sl)
        q.copy_(cur["q"].to(DEV))
        k_new.copy_(cur["k"].to(DEV))
        v_new.copy_(cur["v"].to(DEV))
        slots.copy_(torch.from_numpy(sl).to(DEV))
        ctx.copy_(torch.from_numpy(lens).to(DEV))
        torch.cuda.synchronize()

    def step(kc, vc, out, ws):
        pa.store_kvcache(k_new, v_new, kc, vc, slots)
        pa.decode(q, kc, vc, ctx, bt, scale, out=out, split_tokens=split, workspace=ws)

    draw()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(kc_g, vc_g, out_g, ws_g)
    torch.cuda.synchronize()
    n_rep = 4
    for r in range(n_rep):
        if r > 0:
            draw()
        g.replay()
        torch.cuda.synchronize()
        host.store(cur["k"], cur["v"], cur["slots"])
        if r in (0, n_rep - 1):
            host.check(out_g, cur["q"], cur["lens"], kc_g, what=f"batch {batch} replay {r}")
        step(kc_e, vc_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e).all(), f"replay {r}: eager output not finite"
        assert torch.equal(out_g, out_e), f"replay {r}: graph output differs from the eager calls"
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), f"replay {r}: caches differ"


@pytest.mark.gpu
@pytest.mark.parametrize("batch", [1, 8, 64, 512])
def test_graph_fused_metadata_store_decode_replays(batch):
    """The decode step as the engine runs it, metadata and store in one launch (pa_build_metadata_store) and then
    the balanced decode, captured once and replayed with new cached lengths, queries and K/V."""
    rng = np.random.default_rng(950 + batch)
    mbps = 4 if batch > 64 else 8
    nb = batch * mbps + 4
    perm = rng.permutation(nb).astype(np.int32)
    table = perm[: batch * mbps].reshape(batch, mbps)
    pool_k = _bf16(rng, (nb, BS, HKV, D))
    pool_v = _bf16(rng, (nb, BS, HKV, D))
    host = HostMirror(pool_k, pool_v, table)
    kc_g, vc_g = pool_k.to(DEV), pool_v.to(DEV)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()

    q = torch.empty((batch, HQ, D), dtype=torch.bfloat16, device=DEV)
    k_new = torch.empty((batch, HKV, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    num_cached = torch.empty(batch, dtype=torch.int32, device=DEV)
    num_new = torch.ones(batch, dtype=torch.int32, device=DEV)
    bt = torch.from_numpy(table).to(DEV)
    out_g = torch.empty((batch, HQ, D), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    need = pa.decode_workspace_bytes(batch, HQ, HKV, D, mbps, BS, 0)
    ws_g = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws_g)
    scale = 1.0 / np.sqrt(D)
    cur = {}

    def draw():
        cached = rng.integers(0, mbps * BS, size=batch).astype(np.int32)   # the new token fits the table
        cur.update(q=_bf16(rng, (batch, HQ, D)), k=_bf16(rng, (batch, HKV, D)), v=_bf16(rng, (batch, HKV, D)),
                   lens=cached + 1, slots=_slots(table, cached))
        q.copy_(cur["q"].to(DEV))
        k_new.copy_(cur["k"].to(DEV))
        v_new.copy_(cur["v"].to(DEV))
        num_cached.copy_(torch.from_numpy(cached).to(DEV))
        torch.cuda.synchronize()

    def step(kc, vc, out, ws):
        meta = pa.build_metadata_store(num_cached, num_new, bt, batch, k_new, v_new, kc, vc)
        pa.decode(q, kc, vc, meta["context_lens"], bt, scale, out=out, workspace=ws)
        return meta

    draw()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        meta_g = step(kc_g, vc_g, out_g, ws_g)
    torch.cuda.synchronize()
    n_rep = 4
    for r in range(n_rep):
        if r > 0:
            draw()
        g.replay()
        torch.cuda.synchronize()
        host.store(cur["k"], cur["v"], cur["slots"])
        if r in (0, n_rep - 1):
            assert np.array_equal(meta_g["slot_mapping"].cpu().numpy(), cur["slots"])
            host.check(out_g, cur["q"], cur["lens"], kc_g, what=f"batch {batch} replay {r}")
        meta_e = step(kc_e, vc_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e).all(), f"replay {r}: eager output not finite"
        for key in ("slot_mapping", "context_lens", "positions", "cu_seqlens_k"):
            assert torch.equal(meta_g[key], meta_e[key]), f"replay {r}: {key} differs"
        assert torch.equal(out_g, out_e), f"replay {r}: graph output differs from the eager calls"
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), f"replay {r}: caches differ"


@pytest.mark.gpu
@pytest.mark.parametrize("batch", [1, 8, 64, 512])
def test_graph_decode_append_replays(batch):
    """pa_decode_append (slots from the table, store and attention in the decode's two launches) captured once and
    replayed with new cached lengths, queries and K/V; each replay must equal, bit for bit, the metadata + store
    launch followed by pa_decode run eagerly on a second pool (the same arithmetic over the same lengths), and
    the first and last replays the oracle."""
    rng = np.random.default_rng(970 + batch)
    mbps = 4 if batch > 64 else 8
    nb = batch * mbps + 4
    perm = rng.permutation(nb).astype(np.int32)
    table = perm[: batch * mbps].reshape(batch, mbps)
    pool_k, pool_v = _bf16(rng, (nb, BS, HKV, D)), _bf16(rng, (nb, BS, HKV, D))
    host = HostMirror(pool_k, pool_v, table)
    kc_g, vc_g = pool_k.to(DEV), pool_v.to(DEV)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()

    q = torch.empty((batch, HQ, D), dtype=torch.bfloat16, device=DEV)
    k_new = torch.empty((batch, HKV, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    num_cached = torch.empty(batch, dtype=torch.int32, device=DEV)
    num_new = torch.ones(batch, dtype=torch.int32, device=DEV)
    bt = torch.from_numpy(table).to(DEV)
    out_g = torch.empty((batch, HQ, D), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    need = pa.decode_workspace_bytes(batch, HQ, HKV, D, mbps, BS, 0)
    ws_g = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws_g)
    scale = 1.0 / np.sqrt(D)
    cur = {}

    def draw():
        cached = rng.integers(0, mbps * BS, size=batch).astype(np.int32)
        cur.update(q=_bf16(rng, (batch, HQ, D)), k=_bf16(rng, (batch, HKV, D)), v=_bf16(rng, (batch, HKV, D)),
                   lens=cached + 1, slots=_slots(table, cached))
        q.copy_(cur["q"].to(DEV))
        k_new.copy_(cur["k"].to(DEV))
        v_new.copy_(cur["v"].to(DEV))
        num_cached.copy_(torch.from_numpy(cached).to(DEV))
        torch.cuda.synchronize()

    draw()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.decode_append(q, k_new, v_new, kc_g, vc_g, num_cached, bt, scale, out=out_g, workspace=ws_g,
                         fallback=False)
    torch.cuda.synchronize()
    n_rep = 4
    for r in range(n_rep):
        if r > 0:
            draw()
        g.replay()
        torch.cuda.synchronize()
        host.store(cur["k"], cur["v"], cur["slots"])
        if r in (0, n_rep - 1):
            host.check(out_g, cur["q"], cur["lens"], kc_g, what=f"batch {batch} replay {r}")
        meta = pa.build_metadata_store(num_cached, num_new, bt, batch, k_new, v_new, kc_e, vc_e)
        pa.decode(q, kc_e, vc_e, meta["context_lens"], bt, scale, out=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e).all(), f"replay {r}: eager output not finite"
        assert torch.equal(out_g, out_e), f"replay {r}: graph output differs from store + decode"
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), f"replay {r}: caches differ"


@pytest.mark.gpu
def test_two_streams_at_once_match_sequential_calls():
    """The library keeps no per-call state of its own: decode steps enqueued on two streams at the same time
    (separate caches, outputs and workspaces) give the results of the same calls made one after the other."""
    rng = np.random.default_rng(990)
    B, mbps = 32, 8
    nb = B * mbps + 4

    def setup():
        table = rng.permutation(nb).astype(np.int32)[: B * mbps].reshape(B, mbps)
        kc = _bf16(rng, (nb, BS, HKV, D)).to(DEV)
        vc = _bf16(rng, (nb, BS, HKV, D)).to(DEV)
        q = _bf16(rng, (B, HQ, D)).to(DEV)
        kn = _bf16(rng, (B, HKV, D)).to(DEV)
        vn = _bf16(rng, (B, HKV, D)).to(DEV)
        cached = torch.from_numpy(rng.integers(0, mbps * BS, size=B).astype(np.int32)).to(DEV)
        return dict(table=torch.from_numpy(table).to(DEV), kc=kc, vc=vc, q=q, kn=kn, vn=vn, cached=cached)

    jobs = [setup(), setup()]
    need = pa.decode_workspace_bytes(B, HQ, HKV, D, mbps, BS, 0)
    scale = 1.0 / np.sqrt(D)

    def run(j, out, ws, kc, vc, stream=None):
        pa.decode_append(j["q"], j["kn"], j["vn"], kc, vc, j["cached"], j["table"], scale, out=out, workspace=ws,
                         fallback=False, stream=stream)

    # sequential reference on copies of the caches
    ref = []
    for j in jobs:
        out = torch.empty((B, HQ, D), dtype=torch.float32, device=DEV)
        kc, vc = j["kc"].clone(), j["vc"].clone()
        run(j, out, torch.empty(need, dtype=torch.uint8, device=DEV), kc, vc)
        torch.cuda.synchronize()
        ref.append((out, kc, vc))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((B, HQ, D), dtype=torch.float32, device=DEV) for _ in jobs]
    wss = [torch.empty(need, dtype=torch.uint8, device=DEV) for _ in jobs]
    torch.cuda.synchronize()
    for _ in range(3):  # repeated: the appended rows are stored again with the same values
        for j, out, ws, st in zip(jobs, outs, wss, streams):
            run(j, out, ws, j["kc"], j["vc"], stream=st)
        torch.cuda.synchronize()
        for (o_ref, kc_ref, vc_ref), out, j in zip(ref, outs, jobs):
            assert torch.equal(out, o_ref)
            assert torch.equal(j["kc"], kc_ref) and torch.equal(j["vc"], vc_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["decode", "prefill_split"])
def test_workspace_contents_do_not_matter(kind):
    """The workspace is scratch: every partial a call reads back it wrote in the same call. A workspace full of
    NaN bytes gives the bit-identical output of a zeroed one."""
    rng = np.random.default_rng(995)
    mbps = 40 if kind == "prefill_split" else 8
    B = 1 if kind == "prefill_split" else 48
    nb = B * mbps + 4
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[: B * mbps].reshape(B, mbps)).to(DEV)
    kc = _bf16(rng, (nb, BS, HKV, D)).to(DEV)
    vc = _bf16(rng, (nb, BS, HKV, D)).to(DEV)
    scale = 1.0 / np.sqrt(D)
    outs = []
    for fill in (0x00, 0xFF):  # 0xFFFF... is a NaN in every float width
        if kind == "decode":
            lens = torch.from_numpy(np.random.default_rng(7).integers(1, mbps * BS + 1, size=B).astype(np.int32))
            lens = lens.to(DEV)
            q = _bf16(np.random.default_rng(8), (B, HQ, D)).to(DEV)
            need = pa.decode_workspace_bytes(B, HQ, HKV, D, mbps, BS, 0)
            ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
            outs.append(pa.decode(q, kc, vc, lens, table, scale, workspace=ws))
        else:
            q_len, k_len = 200, mbps * BS  # 200 rows over 10240 keys: key splits and the merge pass
            q = _bf16(np.random.default_rng(9), (q_len, HQ, D)).to(DEV)
            cu_q = torch.tensor([0, q_len], dtype=torch.int32, device=DEV)
            cu_k = torch.tensor([0, k_len], dtype=torch.int32, device=DEV)
            need = pa.prefill_workspace_bytes(1, HQ, D, q_len, k_len)
            assert need > 0
            ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
            outs.append(pa.prefill_varlen(q, kc, vc, cu_q, cu_k, table, q_len, k_len, scale, workspace=ws))
        torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.gpu
def test_graph_prefill_with_key_splits_replays():
    """The key-split prefill (split count and grids from host sizes only) captured once and replayed with new
    queries and cache contents: every replay equals the eager call bit for bit, and the first and last the
    oracle."""
    rng = np.random.default_rng(996)
    mbps, q_len = 40, 200
    k_len = mbps * BS
    nb = mbps + 4
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[:mbps].reshape(1, mbps)).to(DEV)
    kc = torch.empty((nb, BS, HKV, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    q = torch.empty((q_len, HQ, D), dtype=torch.bfloat16, device=DEV)
    cu_q = torch.tensor([0, q_len], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, k_len], dtype=torch.int32, device=DEV)
    need = pa.prefill_workspace_bytes(1, HQ, D, q_len, k_len)
    ws_g = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws_g)
    out_g = torch.empty((q_len, HQ, D), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    scale = 1.0 / np.sqrt(D)

    cur = {}

    def draw():
        cur.update(k=_bf16(rng, tuple(kc.shape)), v=_bf16(rng, tuple(vc.shape)), q=_bf16(rng, tuple(q.shape)))
        kc.copy_(cur["k"].to(DEV))
        vc.copy_(cur["v"].to(DEV))
        q.copy_(cur["q"].to(DEV))
        torch.cuda.synchronize()

    draw()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.prefill_varlen(q, kc, vc, cu_q, cu_k, table, q_len, k_len, scale, out=out_g, workspace=ws_g)
    torch.cuda.synchronize()
    for r in range(3):
        if r > 0:
            draw()
        g.replay()
        torch.cuda.synchronize()
        if r in (0, 2):
            ref = oracle.prefill_varlen(_bits(cur["q"]), _bits(cur["k"]), _bits(cur["v"]), np.array([0, q_len]),
                                        np.array([0, k_len]), table.cpu().numpy(), scale, "bf16")
            assert_close(out_g, ref, what=f"prefill replay {r}")
        pa.prefill_varlen(q, kc, vc, cu_q, cu_k, table, q_len, k_len, scale, out=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e).all()
        assert torch.equal(out_g, out_e), f"replay {r}"
