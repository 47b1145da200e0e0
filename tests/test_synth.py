"""The seeded input generator: splitmix64 used as a counter generator, checked
against the generator's published definition restated with Python integers
(state += 0x9E3779B97F4A7C15; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
z = (z ^ z>>27) * 0x94D049BB133111EB; z ^ z>>31, all mod 2^64) and its
well-known first output for seed 0; then the value recipes built on it."""
import math

import numpy as np
import torch

import synth

MASK = (1 << 64) - 1


def _reference(seed, n):
    out, state = [], seed & MASK
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_matches_its_definition():
    assert int(synth.splitmix64(0, 1)[0]) & MASK == 0xE220A8397B1DCDAF
    for seed in (0, 1, 12345, synth.seed_of(5, 0, 3), (1 << 64) - 1):
        got = [int(v) & MASK for v in synth.splitmix64(seed, 300)]
        assert got == _reference(seed, 300), seed


def test_uniform_is_top_24_bits():
    u = synth.uniform((4096,), 0.0, 1.0, 77)
    want = np.array([(v >> 40) / 2.0 ** 24 for v in _reference(77, 4096)], dtype=np.float32)
    assert np.array_equal(u.numpy(), want)
    v = synth.uniform((3, 5), -2.0, 6.0, 78)
    assert v.shape == (3, 5) and float(v.min()) >= -2.0 and float(v.max()) < 6.0


def test_normal_is_box_muller_of_two_draws():
    n = 2000
    x = synth.normal((n,), 1.5, 91)
    r = _reference(91, 2 * n)
    want = []
    for i in range(n):
        u1 = ((r[2 * i] >> 11) + 1) * 2.0 ** -53
        u2 = (r[2 * i + 1] >> 11) * 2.0 ** -53
        want.append(math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2) * 1.5)
    want = np.array(want, dtype=np.float64).astype(np.float32)
    got = x.numpy()
    # libm and torch may differ in the last fp64 bit of log / cos: at most one fp32 step apart
    assert np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64)).max() <= 1
    assert np.count_nonzero(got != want) <= 2
    big = synth.normal((1 << 20,), 1.0, 5)
    assert abs(float(big.mean())) < 5e-3 and abs(float(big.std()) - 1.0) < 5e-3
    assert synth.normal((4, 6), 1.0, 5, dtype=torch.bfloat16).dtype == torch.bfloat16


def test_permutation_and_outlier_channels():
    p = synth.permutation(4096, 9)
    assert sorted(p.tolist()) == list(range(4096))
    keys = [(v ^ (1 << 63)) for v in _reference(9, 4096)]        # signed order of the draws
    assert p.tolist() == sorted(range(4096), key=lambda i: keys[i])
    assert torch.equal(synth.mlp_outlier_channels(), synth.permutation(4096, synth.seed_of(3, 0, 9))[:4])
