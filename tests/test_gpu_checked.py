"""The index checker (pa_check_indices) and checked mode (PA_CHECKED=1) on the GPU.

The path trusts its indices; the checker reads only the index arrays and reports, per kind, how many entries
would send the path out of bounds and the first of them. Expected reports are the rules of include/pa.h
written out here in NumPy. Invalid arrays reach only the checker and the metadata kernel, whose table reads stop
at the row: in checked mode the store, prefill and decode calls raise before launching, which the tests verify
by the caches and outputs staying untouched.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_111_amd as pa
from harness import DEV, i32

pytestmark = pytest.mark.gpu

NB, BS, MBPS = 40, 16, 6          # pool of 640 slots; rows of 6 blocks (96 keys)


def _expected(num_blocks, block_size, slots=None, table=None, lens=None, cu_q=None, cu_k=None, num_tokens=None):
    """The report the rules give, as {kind: (count, first)}."""
    rep = {k: [0, None] for k in pa.CHECK_KINDS}

    def flag(kind, idx):
        rep[kind][0] += 1
        rep[kind][1] = idx if rep[kind][1] is None else min(rep[kind][1], idx)

    if slots is not None:
        for t, sl in enumerate(slots):
            if sl >= num_blocks * block_size:
                flag("slot", t)
    if cu_q is not None or cu_k is not None:
        batch = len(cu_q if cu_q is not None else cu_k) - 1
        for i in range(batch + 1):
            bad = False
            if cu_q is not None:
                bad |= cu_q[0] != 0 if i == 0 else cu_q[i] < cu_q[i - 1]
                if i == batch:
                    bad |= cu_q[batch] != num_tokens
            if cu_k is not None:
                bad |= cu_k[0] != 0 if i == 0 else cu_k[i] < cu_k[i - 1]
            if bad:
                flag("cu", i)
    if lens is not None or cu_k is not None:
        mbps = table.shape[1]
        batch = len(lens) if lens is not None else len(cu_k) - 1
        for s in range(batch):
            k_len = int(lens[s]) if lens is not None else int(cu_k[s + 1]) - int(cu_k[s])
            if k_len < 0 or k_len > mbps * block_size:
                flag("len", s)
                continue
            if cu_q is not None and cu_k is not None and int(cu_q[s + 1]) - int(cu_q[s]) > k_len:
                flag("q_gt_k", s)
            for b in range(-(-k_len // block_size)):
                if not 0 <= table[s, b] < num_blocks:
                    flag("table", s * mbps + b)
    return {k: tuple(v) for k, v in rep.items()}


def _got(rep):
    return {k: (v["count"], v["first"]) for k, v in rep.items()}


def _table(rng, batch, fill_unused=-7):
    t = np.full((batch, MBPS), fill_unused, np.int32)
    ids = rng.permutation(NB).astype(np.int32)
    for s in range(batch):
        t[s] = ids[(s * MBPS) % (NB - MBPS):][:MBPS]
    return t


def test_valid_arrays_report_nothing():
    rng = np.random.default_rng(1)
    table = _table(rng, 4)
    lens = np.array([1, 96, 40, 17], np.int32)
    table[0, 1:] = -1                     # entries past a sequence's length are never looked at
    slots = np.array([-1, 0, 639, 300], np.int32)
    rep = pa.check_indices(NB, BS, slot_mapping=i32(slots), block_table=i32(table), context_lens=i32(lens))
    assert all(v["count"] == 0 and v["first"] is None for v in rep.values()), rep
    cu_q = np.array([0, 1, 30, 30, 47], np.int32)
    cu_k = np.array([0, 1, 97, 137, 154], np.int32)
    rep = pa.check_indices(NB, BS, num_tokens=47, block_table=i32(table), cu_seqlens_q=i32(cu_q),
                           cu_seqlens_k=i32(cu_k))
    assert all(v["count"] == 0 for v in rep.values()), rep


def test_each_kind_is_counted_with_its_first_index():
    rng = np.random.default_rng(2)
    batch = 300
    table = _table(rng, batch)
    lens = rng.integers(1, MBPS * BS + 1, batch).astype(np.int32)
    lens[[5, 77]] = MBPS * BS + 1         # beyond the row
    lens[150] = -3
    used = -(-lens.clip(0) // BS)
    table[9, used[9] - 1] = NB            # last used entry out of range
    table[200, 0] = -1
    table[11, MBPS - 1] = 10 ** 6 if used[11] < MBPS else table[11, MBPS - 1]   # unused entry: not an error
    slots = rng.integers(-1, NB * BS, 5000).astype(np.int32)
    slots[[17, 4000]] = NB * BS
    slots[2500] = 2 ** 31 - 1
    rep = pa.check_indices(NB, BS, slot_mapping=i32(slots), block_table=i32(table), context_lens=i32(lens))
    want = _expected(NB, BS, slots=slots, table=table, lens=lens)
    assert _got(rep) == want
    assert want["slot"] == (3, 17) and want["len"] == (3, 5) and want["table"][0] == 2


def test_prefill_arrays():
    rng = np.random.default_rng(3)
    table = _table(rng, 5)
    q_len = np.array([3, 10, 0, 4, 8])
    k_len = np.array([3, 96, 5, 2, 20])   # sequence 3 has more new rows than keys
    cu_q = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_len)]).astype(np.int32)
    for name, cq, ck, T in (("as given", cu_q, cu_k, int(cu_q[-1])),
                            ("wrong total", cu_q, cu_k, int(cu_q[-1]) + 1),
                            ("decreasing", cu_q, np.array([0, 3, 99, 90, 106, 126], np.int32), int(cu_q[-1])),
                            ("not from 0", np.array([1, 3, 13, 13, 17, 25], np.int32), cu_k, 25)):
        rep = pa.check_indices(NB, BS, num_tokens=T, block_table=i32(table), cu_seqlens_q=i32(cq),
                               cu_seqlens_k=i32(ck))
        want = _expected(NB, BS, table=table, cu_q=cq, cu_k=ck, num_tokens=T)
        print(f"[case] prefill {name}: {want}", flush=True)
        assert _got(rep) == want, name
        assert want["q_gt_k"][0] >= (1 if name == "as given" else 0)


def test_metadata_gives_no_slot_outside_the_row():
    """A position beyond a sequence's table row (or a negative one) gets slot -1 and no table read."""
    table = np.arange(2 * MBPS, dtype=np.int32).reshape(2, MBPS)
    cached = np.array([MBPS * BS - 2, -5], np.int32)
    new = np.array([4, 2], np.int32)
    meta = pa.build_metadata(i32(cached), i32(new), i32(table), 6, NB, BS)
    slots = meta["slot_mapping"].cpu().numpy()
    pos = meta["positions"].cpu().numpy()
    np.testing.assert_array_equal(pos, [MBPS * BS - 2, MBPS * BS - 1, MBPS * BS, MBPS * BS + 1, -5, -4])
    np.testing.assert_array_equal(slots[:2], [table[0, MBPS - 1] * BS + BS - 2, table[0, MBPS - 1] * BS + BS - 1])
    np.testing.assert_array_equal(slots[2:], [-1, -1, -1, -1])


def test_checked_mode_raises_before_launching(monkeypatch):
    monkeypatch.setenv("PA_CHECKED", "1")
    rng = np.random.default_rng(4)
    Hq, Hkv, D = 4, 2, 128
    kc = torch.from_numpy(rng.standard_normal((NB, BS, Hkv, D), dtype=np.float32)).to(DEV).bfloat16()
    vc = kc.clone()
    kc0 = kc.clone()
    k = torch.ones((3, Hkv, D), dtype=torch.bfloat16, device=DEV)
    # store: one slot past the pool
    with pytest.raises(pa.PAIndexError) as e:
        pa.store_kvcache(k, k, kc, vc, i32([5, NB * BS, 7]))
    assert e.value.report["slot"] == {"count": 1, "first": 1}
    assert torch.equal(kc, kc0), "nothing may be stored when the call is refused"
    # a valid store goes through in checked mode
    pa.store_kvcache(k, k, kc, vc, i32([5, -1, 7]))
    torch.cuda.synchronize()
    assert torch.equal(kc.view(NB * BS, Hkv, D)[5], k[0])
    # decode: a used table entry out of range
    table = _table(rng, 2)
    table[1, 0] = NB + 3
    q = torch.ones((2, Hq, D), dtype=torch.bfloat16, device=DEV)
    out = torch.full((2, Hq, D), 7.0, device=DEV)
    with pytest.raises(pa.PAIndexError) as e:
        pa.decode(q, kc, vc, i32([20, 30]), i32(table), 0.1, out=out)
    assert e.value.report["table"] == {"count": 1, "first": MBPS}
    assert bool((out == 7.0).all())
    # prefill: more new rows than keys
    with pytest.raises(pa.PAIndexError) as e:
        pa.prefill_varlen(torch.ones((5, Hq, D), dtype=torch.bfloat16, device=DEV), kc, vc, i32([0, 2, 5]),
                          i32([0, 2, 4]), i32(_table(rng, 2)), 3, 2, 0.1)
    assert e.value.report["q_gt_k"]["count"] == 1
    # metadata + store: the new tokens run past the table row, so nothing is stored
    with pytest.raises(pa.PAIndexError) as e:
        pa.build_metadata_store(i32([MBPS * BS - 1]), i32([3]), i32(_table(rng, 1)), 3, k, k, kc, vc)
    assert e.value.report["len"]["count"] == 1
    rows = torch.arange(NB * BS, device=DEV)
    kept = (rows != 5) & (rows != 7)      # the two rows of the valid store above
    assert torch.equal(kc.view(NB * BS, Hkv, D)[kept], kc0.view(NB * BS, Hkv, D)[kept])
    assert torch.equal(kc.view(NB * BS, Hkv, D)[7], k[2])


def test_checked_mode_decode_append(monkeypatch):
    """pa_decode_append in checked mode: the binding validates the metadata and lengths it derives, so a table
    whose entry for the new token is out of range raises before anything is stored or computed."""
    monkeypatch.setenv("PA_CHECKED", "1")
    rng = np.random.default_rng(5)
    Hq, Hkv, D = 4, 2, 128
    bs = 32
    nb = 20
    kc = torch.from_numpy(rng.standard_normal((nb, bs, Hkv, D), dtype=np.float32)).to(DEV).bfloat16()
    vc = kc.clone()
    kc0 = kc.clone()
    table = np.arange(2 * 4, dtype=np.int32).reshape(2, 4)
    table[1, 2] = nb + 1                      # the block of sequence 1's new token (position 70)
    q = torch.ones((2, Hq, D), dtype=torch.bfloat16, device=DEV)
    k_new = torch.full((2, Hkv, D), 3.0, dtype=torch.bfloat16, device=DEV)
    out = torch.full((2, Hq, D), 7.0, device=DEV)
    with pytest.raises(pa.PAIndexError):
        pa.decode_append(q, k_new, k_new, kc, vc, i32([10, 70]), i32(table), 0.1, out=out)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc0) and bool((out == 7.0).all())
    # the same call with a valid table stores both rows and computes the output
    table[1, 2] = 9
    pa.decode_append(q, k_new, k_new, kc, vc, i32([10, 70]), i32(table), 0.1, out=out)
    torch.cuda.synchronize()
    flat = kc.view(nb * bs, Hkv, D)
    assert torch.equal(flat[table[0, 0] * bs + 10], k_new[0]) and torch.equal(flat[9 * bs + 70 - 64], k_new[1])
    assert torch.isfinite(out).all()
