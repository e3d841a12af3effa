"""Pins of the oracle's pre-attention step (oracle/rope.py) to facts outside its own code: closed forms of RMSNorm,
the rotate-half convention on unit vectors, the geometry of rotations (norm kept, angles add, scores depend only
on the position difference), the placement of the stored rows, and bf16 rounding against torch. Planted mistakes
(interleaved pairs, a flipped sine, a sum instead of a mean, an off-by-one position) each fail at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.rope as orope
from workloads import build_rope_inputs, encode_values


def _table(angles: np.ndarray) -> np.ndarray:
    """Rotary table rows for explicit angles [P, D/2] (float64): cos in the first half, sin in the second."""
    return np.concatenate([np.cos(angles), np.sin(angles)], axis=1)


# ------------------------------------------------------------------------------------------ RMSNorm


def test_rms_norm_of_a_constant_vector():
    x = np.full((1, 8), 3.0)
    np.testing.assert_array_equal(orope.rms_norm(x, np.ones(8), 0.0), np.ones((1, 8)))
    eps = 0.5
    np.testing.assert_allclose(orope.rms_norm(x, np.ones(8), eps), np.full((1, 8), 3.0 / np.sqrt(9.0 + eps)),
                               rtol=1e-15)


def test_rms_norm_unit_mean_square_scale_invariance_and_weight():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 16))
    y = orope.rms_norm(x, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orope.rms_norm(7.5 * x, np.ones(16), 0.0), y, rtol=1e-13)
    w = rng.standard_normal(16)
    np.testing.assert_allclose(orope.rms_norm(x, w, 1e-6), orope.rms_norm(x, np.ones(16), 1e-6) * w, rtol=1e-13)


# ------------------------------------------------------------------------------------------ rotation


def test_rotate_half_convention_on_unit_vectors():
    """D = 4: frequency i rotates the pair (x[i], x[i + 2]); e0 -> (cos a, 0, sin a, 0), e2 -> (-sin a, 0, cos a, 0),
    e1 -> (0, cos b, 0, sin b)."""
    a, b = 0.7, -1.9
    cos, sin = np.array([np.cos(a), np.cos(b)]), np.array([np.sin(a), np.sin(b)])
    eye = np.eye(4)
    np.testing.assert_allclose(orope.rope_rotate_half(eye[0], cos, sin), [np.cos(a), 0, np.sin(a), 0], atol=1e-15)
    np.testing.assert_allclose(orope.rope_rotate_half(eye[2], cos, sin), [-np.sin(a), 0, np.cos(a), 0], atol=1e-15)
    np.testing.assert_allclose(orope.rope_rotate_half(eye[1], cos, sin), [0, np.cos(b), 0, np.sin(b)], atol=1e-15)


def test_position_zero_is_the_identity_and_positions_index_the_table():
    d = build_rope_inputs(11, 6, 4, 2, 16, "f32", 32, positions=[0, 0, 1, 5, 31, 0])
    cs = d["cos_sin"]
    np.testing.assert_array_equal(cs[0, :8], 1.0)
    np.testing.assert_array_equal(cs[0, 8:], 0.0)
    x = np.random.default_rng(4).standard_normal((6, 2, 16))
    w = np.ones(16)
    y = orope.norm_rope(x, w, 0.0, d["positions"], cs)
    n = orope.rms_norm(x, w, 0.0)
    for t in (0, 1, 5):
        np.testing.assert_allclose(y[t], n[t], rtol=1e-15)
    # token 3 at position 5 uses row 5 of the table
    row = cs[5].astype(np.float64)
    np.testing.assert_allclose(y[3], orope.rope_rotate_half(n[3], row[:8], row[8:]), rtol=1e-15)


def test_rotation_keeps_pair_norms_and_angles_add():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 3, 32))
    a = rng.uniform(-4, 4, size=(7, 1, 16))
    b = rng.uniform(-4, 4, size=(7, 1, 16))
    ra = orope.rope_rotate_half(x, np.cos(a), np.sin(a))
    pair = lambda z: z[..., :16] ** 2 + z[..., 16:] ** 2  # noqa: E731
    np.testing.assert_allclose(pair(ra), pair(x), rtol=1e-12)
    rab = orope.rope_rotate_half(ra, np.cos(b), np.sin(b))
    np.testing.assert_allclose(rab, orope.rope_rotate_half(x, np.cos(a + b), np.sin(a + b)), atol=1e-12)


def test_scores_depend_only_on_the_position_difference():
    """With angles linear in the position, q at m and k at n give the same dot product as at m+s, n+s."""
    D = 64
    inv_freq = 10000.0 ** (-np.arange(0, D, 2) / D)
    cs = _table(np.arange(256)[:, None] * inv_freq[None, :])
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    one = np.ones(D)
    for m, n, s in ((10, 3, 100), (0, 0, 77), (5, 40, 200)):
        d0 = np.sum(orope.norm_rope(q, one, 0.0, [m], cs) * orope.norm_rope(k, one, 0.0, [n], cs))
        d1 = np.sum(orope.norm_rope(q, one, 0.0, [m + s], cs) * orope.norm_rope(k, one, 0.0, [n + s], cs))
        np.testing.assert_allclose(d1, d0, rtol=1e-9, atol=1e-9)


# ------------------------------------------------------------------------------------------ store and rounding


def test_norm_rope_store_places_rotated_keys_and_copies_values():
    T, Hkv, D, nb, bs = 5, 2, 16, 4, 4
    d = build_rope_inputs(12, T, 4, Hkv, D, "bf16", 64)
    kc = np.full((nb, bs, Hkv, D), 7, dtype=np.uint16)
    vc = np.full((nb, bs, Hkv, D), 9, dtype=np.uint16)
    slots = np.array([3, 14, -1, 0, 9], dtype=np.int32)
    k_rot, q_rot = orope.norm_rope_store(d["k"], d["v"], d["k_weight"], d["eps"], d["positions"], d["cos_sin"],
                                         kc, vc, slots, "bf16", q=d["q"], q_weight=d["q_weight"])
    kf, vf = kc.reshape(nb * bs, Hkv, D), vc.reshape(nb * bs, Hkv, D)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        np.testing.assert_array_equal(kf[s], orope.round_to(k_rot[t], "bf16"))
        np.testing.assert_array_equal(vf[s], d["v"][t])
    untouched = np.setdiff1d(np.arange(nb * bs), slots[slots >= 0])
    assert np.all(kf[untouched] == 7) and np.all(vf[untouched] == 9)
    assert q_rot.shape == (T, 4, D)
    kw = oracle.to_f64(d["k_weight"], "bf16")
    np.testing.assert_allclose(k_rot, orope.norm_rope(oracle.to_f64(d["k"], "bf16"), kw, d["eps"], d["positions"],
                                                      d["cos_sin"]), rtol=1e-15)


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096),
                        1.0 + np.array([2.0 ** -8, 3 * 2.0 ** -8, -(2.0 ** -9)])])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orope.round_to(x, "bf16"), ref)
    # round half to even at the two midpoints above 1.0: 1 + 2^-8 -> 1.0, 1 + 3 * 2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(orope.round_to(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]), "bf16"),
                                  encode_values(np.array([1.0, 1.0 + 2.0 ** -6]), "bf16"))


# ------------------------------------------------------------------------------------------ mutation checks


def _interleaved(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x2 * cos + x1 * sin
    return out


def _flipped_sine(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    return np.concatenate([x[..., :h] * cos + x[..., h:] * sin, x[..., h:] * cos - x[..., :h] * sin], axis=-1)


def _sum_norm(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * w


@pytest.mark.parametrize("kind", ["interleaved", "flipped_sine", "sum_norm", "position_plus_one"])
def test_pins_catch_planted_mistakes(monkeypatch, kind):
    if kind == "interleaved":
        monkeypatch.setattr(orope, "rope_rotate_half", _interleaved)
    elif kind == "flipped_sine":
        monkeypatch.setattr(orope, "rope_rotate_half", _flipped_sine)
    elif kind == "sum_norm":
        monkeypatch.setattr(orope, "rms_norm", _sum_norm)
    else:
        real = orope.norm_rope

        def shifted(x, w, eps, positions, cos_sin):
            return real(x, w, eps, np.minimum(np.asarray(positions) + 1, len(cos_sin) - 1), cos_sin)

        monkeypatch.setattr(orope, "norm_rope", shifted)
    failures = 0
    for test in (test_rms_norm_of_a_constant_vector, test_rms_norm_unit_mean_square_scale_invariance_and_weight,
                 test_rotate_half_convention_on_unit_vectors,
                 test_position_zero_is_the_identity_and_positions_index_the_table):
        try:
            test()
        except AssertionError:
            failures += 1
    assert failures >= 1
