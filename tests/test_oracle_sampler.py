"""Pins of the oracle's sampler (oracle/sampler.py) to facts outside its own code.

The pages give the method (temperature, softmax, Gumbel-max), not numbers. The generator is pinned by the
known-answer vectors its authors publish with their reference implementation (Random123, file kat_vectors,
entries "philox4x32 10"), which fix the word order, both multipliers, the key schedule and the round count. The
sampler is pinned by the distribution of the sampled token against softmax(l / T) (chi-square
over many independent rows), the limits and identities of the temperature (greedy at 0, l / T at 1 equals the
sample at T), the uniformity and avalanche of the generator, exact representability of the uniforms, and the
tie rule. A flipped Gumbel sign, a temperature that multiplies, plain exponential noise in place of the Gumbel
variable, and a counter that ignores the row each fail a pin.
"""

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.sampler as osamp


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


# ------------------------------------------------------------------------------------------ generator identity

# Philox4x32-10 known answers: (counter words 0..3, key words 0..1) -> output words 0..3. Source: the known-answer
# vectors distributed with Random123 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
# SC 2011), entries for philox4x32 with 10 rounds: an all-zero input, an all-ones input, and the digits of pi.
PHILOX4X32_10_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX4X32_10_KAT)
def test_philox_matches_published_known_answers(ctr, key, want):
    got = osamp.philox4x32_10(*(np.array([c], dtype=np.uint64) for c in ctr), key[0], key[1])
    assert tuple(int(w[0]) for w in got) == want


def test_philox_known_answers_in_a_batch():
    """The vectorised form gives each lane its own answer (no mixing across array elements)."""
    ctr = np.array([c for c, _, _ in PHILOX4X32_10_KAT], dtype=np.uint64).T
    for j, (_, key, want) in enumerate(PHILOX4X32_10_KAT):
        got = osamp.philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1])
        assert tuple(int(w[j]) for w in got) == want


@pytest.mark.parametrize("mistake", ["swap_outputs", "key_bump", "nine_rounds"])
def test_planted_generator_mistakes_fail_the_known_answers(mistake, monkeypatch):
    """A generator with its output words permuted, a wrong key-bump constant or one round short (each of which
    the statistical pins below would pass) misses the published answers."""
    if mistake == "swap_outputs":
        real = osamp.philox4x32_10

        def gen(*a):
            x0, x1, x2, x3 = real(*a)
            return x1, x0, x3, x2
    elif mistake == "key_bump":
        monkeypatch.setattr(osamp, "W1", 0xBB67AE86)
        gen = osamp.philox4x32_10
    else:
        def gen(c0, c1, c2, c3, k0, k1):
            # nine rounds: undo the tenth by running the definition with the round count changed
            x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
            ka, kb = np.uint64(k0), np.uint64(k1)
            for r in range(9):
                if r:
                    ka = (ka + np.uint64(osamp.W0)) & np.uint64(osamp.MASK32)
                    kb = (kb + np.uint64(osamp.W1)) & np.uint64(osamp.MASK32)
                p0, p1 = x0 * np.uint64(osamp.M0), x2 * np.uint64(osamp.M1)
                x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ ka, p1 & np.uint64(osamp.MASK32),
                                  (p0 >> np.uint64(32)) ^ x3 ^ kb, p0 & np.uint64(osamp.MASK32))
            return tuple(w.astype(np.uint32) for w in (x0, x1, x2, x3))
    misses = 0
    for ctr, key, want in PHILOX4X32_10_KAT:
        got = gen(*(np.array([c], dtype=np.uint64) for c in ctr), key[0], key[1])
        misses += tuple(int(w[0]) for w in got) != want
    assert misses == len(PHILOX4X32_10_KAT)


# ------------------------------------------------------------------------------------------ distribution


def _frequency_test(logits, T, n_rows=200_000, seed=77, offset=3):
    toks, _ = osamp.sample(np.broadcast_to(logits.astype(np.float32), (n_rows, logits.size)),
                           np.full(n_rows, T), seed, offset)
    counts = np.bincount(toks, minlength=logits.size)
    expected = _softmax(logits.astype(np.float64) / T) * n_rows
    return stats.chisquare(counts, expected).pvalue


@pytest.mark.parametrize("T", [1.0, 0.6, 2.5])
def test_sampled_tokens_follow_softmax_of_logits_over_temperature(T):
    logits = np.array([1.0, -0.5, 2.0, 0.0, 1.5, -2.0])
    assert _frequency_test(logits, T) > 1e-4


def test_temperature_zero_is_greedy_and_ties_go_to_the_lower_index():
    logits = np.array([[0.5, 3.0, -1.0, 3.0], [7.0, 7.0, 7.0, 1.0]], dtype=np.float32)
    toks, _ = osamp.sample(logits, [0.0, 0.0], 1, 0)
    np.testing.assert_array_equal(toks, [1, 0])


def test_small_temperature_picks_the_largest_logit():
    rng = np.random.default_rng(9)
    logits = rng.permutation(np.arange(50, dtype=np.float32))[None, :].repeat(64, 0)  # spaced by 1
    toks, _ = osamp.sample(logits, np.full(64, 1e-3), 5, 11)
    np.testing.assert_array_equal(toks, np.argmax(logits, axis=1))  # noise is within [-2.9, 16.7], x 1e-3 < 1


def test_temperature_scales_the_logits():
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((32, 1000))
    for T in (0.7, 1.9):
        a, _ = osamp.sample(logits, np.full(32, T), 3, 4, dtype=np.float64)
        b, _ = osamp.sample(logits / T, np.full(32, 1.0), 3, 4, dtype=np.float64)
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------------------------------ generator


def test_uniforms_are_exact_odd_multiples_strictly_inside_the_unit_interval():
    u = osamp.uniforms(np.arange(8), 4096, 123, 0)
    assert u.dtype == np.float32 and np.all(u > 0) and np.all(u < 1)
    k = u.astype(np.float64) * 2.0 ** 24
    np.testing.assert_array_equal(k, np.round(k))
    assert np.all(np.round(k) % 2 == 1)


def test_uniforms_are_uniform_and_streams_differ():
    u = osamp.uniforms(np.arange(64), 16384, 2024, 5).reshape(-1)
    counts = np.histogram(u, bins=256, range=(0.0, 1.0))[0]
    assert stats.chisquare(counts).pvalue > 1e-4
    assert stats.kstest(u[:200_000], "uniform").pvalue > 1e-4
    # different row, offset or seed -> unrelated streams
    base = osamp.uniforms([0], 65536, 1, 0)[0]
    for other in (osamp.uniforms([1], 65536, 1, 0)[0], osamp.uniforms([0], 65536, 1, 1)[0],
                  osamp.uniforms([0], 65536, 2, 0)[0]):
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.02
        assert np.mean(base == other) < 1e-3


def test_generator_outputs_are_distinct_and_avalanche():
    n = 1 << 17
    w = osamp.philox4x32_10(np.arange(n), np.zeros(n), np.zeros(n), np.zeros(n), 0, 0)
    packed = {(int(a), int(b), int(c), int(d)) for a, b, c, d in zip(*w)}
    assert len(packed) == n
    bits = np.unpackbits(np.stack(w, axis=1).view(np.uint8), axis=1)
    assert abs(bits.mean() - 0.5) < 0.002
    # flipping one counter bit changes about half of the 128 output bits
    w2 = osamp.philox4x32_10(np.arange(n) ^ 1, np.zeros(n), np.zeros(n), np.zeros(n), 0, 0)
    diff = np.unpackbits((np.stack(w, axis=1) ^ np.stack(w2, axis=1)).view(np.uint8), axis=1).sum(axis=1)
    assert abs(diff.mean() - 64) < 1.0


# ------------------------------------------------------------------------------------------ mutation checks


@pytest.mark.parametrize("kind", ["gumbel_sign", "temperature_multiplies", "exponential_noise", "row_ignored"])
def test_pins_catch_planted_mistakes(monkeypatch, kind):
    real_uniforms = osamp.uniforms
    if kind == "gumbel_sign":
        def f(logits, temperatures, u, dtype=np.float32):
            g = -np.log(-np.log(np.asarray(u, dtype=dtype)))
            t = np.asarray(temperatures, dtype=dtype).reshape(-1, 1)
            return (np.asarray(logits, dtype=dtype) / t - g).astype(dtype)
        monkeypatch.setattr(osamp, "gumbel_scores", f)
    elif kind == "temperature_multiplies":
        def f(logits, temperatures, u, dtype=np.float32):
            g = -np.log(-np.log(np.asarray(u, dtype=dtype)))
            t = np.asarray(temperatures, dtype=dtype).reshape(-1, 1)
            return (np.asarray(logits, dtype=dtype) * t + g).astype(dtype)
        monkeypatch.setattr(osamp, "gumbel_scores", f)
    elif kind == "exponential_noise":
        def f(logits, temperatures, u, dtype=np.float32):
            t = np.asarray(temperatures, dtype=dtype).reshape(-1, 1)
            return (np.asarray(logits, dtype=dtype) / t - np.log(np.asarray(u, dtype=dtype))).astype(dtype)
        monkeypatch.setattr(osamp, "gumbel_scores", f)
    else:
        monkeypatch.setattr(osamp, "uniforms", lambda rows, vocab, seed, offset:
                            real_uniforms(np.zeros_like(np.atleast_1d(rows)), vocab, seed, offset))
    failures = 0
    for test in (lambda: test_sampled_tokens_follow_softmax_of_logits_over_temperature(0.6),
                 test_uniforms_are_uniform_and_streams_differ):
        try:
            test()
        except AssertionError:
            failures += 1
    assert failures >= 1
