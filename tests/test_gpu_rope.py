"""The fused pre-attention step on the GPU (pa_norm_rope_store_kvcache) against the oracle (oracle/rope.py).

Stored keys and rotated queries are fp32 arithmetic rounded to the storage type; they must lie within half a
unit in the last place of the storage type of the oracle's float64 value, plus the fp32 error: the sum of D
squares carries a relative error up to D * 2^-24 (halved by the square root), the scaling, weight and rotation a
few more 2^-24, all relative to the size of the element's rotation pair (which the rotation keeps), so the
allowance is (D + 8) * 2^-24 * |pair|.
Values are bit copies; every cache slot not written keeps its bits; negative slots store nothing.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.rope as orope
import paged_kv_cache_111_amd as pa
from harness import DEV
from workloads import build_rope_inputs

CASES = [
    # T, Hq, Hkv, D, dtype, block_size, max_position
    (64, 16, 8, 128, "bf16", 256, 4096),      # a decode step at the Qwen3-0.6B shape
    (2048, 32, 8, 128, "bf16", 256, 32768),   # a prefill chunk at the Qwen3-8B shape
    (13, 4, 2, 16, "f32", 4, 64),             # the tiny plumbing shape
    (37, 8, 1, 64, "bf16", 16, 512),
    (21, 12, 4, 256, "bf16", 32, 1024),
    (9, 8, 8, 32, "f32", 8, 128),
]


def _ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    bits = 7 if dtype == "bf16" else 23
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - bits)


def _to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _to_f64(t, dtype):
    if dtype == "bf16":
        return oracle.to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.cpu().numpy().astype(np.float64)


def _check_close(got, ref, dtype, what):
    D = ref.shape[-1]
    pair = np.sqrt(ref[..., : D // 2] ** 2 + ref[..., D // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    tol = 0.5 * _ulp(ref, dtype) + (D + 8) * 2.0 ** -24 * pair + 1e-12
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"{what}: worst excess {np.max(err - tol):.3g} (max err {np.max(err):.3g})"


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("with_q", [True, False])
def test_norm_rope_store_matches_oracle(case, with_q):
    T, Hq, Hkv, D, dt, bs, maxp = CASES[case]
    d = build_rope_inputs(400 + case, T, Hq, Hkv, D, dt, maxp)
    rng = np.random.default_rng(500 + case)
    nb = max(4, 2 * T // bs + 2)
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    slots[rng.random(T) < 0.1] = -1                      # some tokens store nothing
    store_t = np.uint16 if dt == "bf16" else np.float32
    kc0 = rng.integers(0, 2 ** 16, size=(nb, bs, Hkv, D)).astype(np.uint16) if dt == "bf16" else \
        rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    vc0 = kc0[::-1].copy()
    kc, vc = _to_dev(kc0, dt), _to_dev(vc0, dt)
    q_out = pa.norm_rope_store_kvcache(
        _to_dev(d["k"], dt), _to_dev(d["v"], dt), kc, vc, torch.from_numpy(slots).to(DEV),
        _to_dev(d["k_weight"], dt), torch.from_numpy(d["positions"]).to(DEV), torch.from_numpy(d["cos_sin"]).to(DEV),
        d["eps"], q=_to_dev(d["q"], dt) if with_q else None, q_norm_weight=_to_dev(d["q_weight"], dt))
    torch.cuda.synchronize()
    print(f"[case] rope case {case} T={T} Hq={Hq} Hkv={Hkv} D={D} {dt} q={with_q}", flush=True)

    ok_kc, ok_vc = kc0.copy(), vc0.copy()
    k_rot, q_rot = orope.norm_rope_store(d["k"], d["v"], d["k_weight"], d["eps"], d["positions"], d["cos_sin"],
                                         ok_kc, ok_vc, slots, dt, q=d["q"] if with_q else None,
                                         q_weight=d["q_weight"])
    got_kc = kc.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else kc.cpu().numpy()
    got_vc = vc.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else vc.cpu().numpy()
    # values and every slot not written: bit for bit
    np.testing.assert_array_equal(got_vc.view(store_t), ok_vc.view(store_t))
    written = np.zeros(nb * bs, dtype=bool)
    written[slots[slots >= 0]] = True
    flat_got = got_kc.reshape(nb * bs, Hkv, D)
    np.testing.assert_array_equal(flat_got[~written], kc0.reshape(nb * bs, Hkv, D)[~written])
    # rotated keys at their slots, against float64
    sel = slots >= 0
    got_k = oracle.to_f64(flat_got[slots[sel]], dt)
    _check_close(got_k, k_rot[sel], dt, "stored keys")
    if with_q:
        _check_close(_to_f64(q_out, dt), q_rot, dt, "rotated queries")
