"""Input generator checks (CPU): bf16 rounding, determinism per seed, and
the structure the workloads promise."""

import numpy as np

from means_nearest_centroid_amd import workloads as W


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_bf16_round_to_nearest_even():
    # (float32 bits, expected bf16 bits); the float32 value is exactly
    # representable, so each case states its rounding by hand.
    cases = [
        (0x3F800000, 0x3F80),   # 1.0 exact
        (0x3F808000, 0x3F80),   # 1 + 2^-8: halfway, even neighbour below
        (0x3F818000, 0x3F82),   # 1 + 3*2^-8: halfway, even neighbour above
        (0x3F808001, 0x3F81),   # just above halfway rounds up
        (0x3F807FFF, 0x3F80),   # just below halfway rounds down
        (0xBF808000, 0xBF80),   # negative halfway, to even
        (0xBF818000, 0xBF82),
        (0x7F7FFFFF, 0x7F80),   # largest float32 rounds past the largest bf16: +inf
        (0x7F7F7FFF, 0x7F7F),   # largest bf16 stays
        (0x7F800000, 0x7F80),   # +inf
        (0xFF800000, 0xFF80),   # -inf
        (0x00000000, 0x0000),   # +0
        (0x80000000, 0x8000),   # -0 keeps its sign
        (0x00018000, 0x0002),   # denormal halfway, to even (0x0001 odd -> 0x0002)
        (0x00008000, 0x0000),   # smallest denormal halfway: to even zero
    ]
    got = W.f32_to_bf16_bits(f32([c[0] for c in cases]))
    assert got.tolist() == [c[1] for c in cases]


def test_bf16_nan_stays_nan_with_sign():
    got = W.f32_to_bf16_bits(f32([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF]))
    assert all((g & 0x7F80) == 0x7F80 and (g & 0x007F) != 0 for g in got.tolist())
    assert (got[1] & 0x8000) and not (got[0] & 0x8000)


def test_bf16_round_trip_is_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(b)
    finite = np.isfinite(f)
    assert np.array_equal(W.f32_to_bf16_bits(f[finite]), b[finite])


def test_generator_is_deterministic_per_seed():
    a = W.gaussian_mixture(300, 64, 40, 17, return_parts=True)
    b = W.gaussian_mixture(300, 64, 40, 17, return_parts=True)
    c = W.gaussian_mixture(300, 64, 40, 29)
    assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2]))
    assert not np.array_equal(a[0], c[0])
    assert a[0].dtype == np.uint16 and a[0].shape == (300, 64) and a[1].shape == (40, 64)


def test_sweep_shapes_are_the_pages_thirteen():
    assert len(W.SWEEP_SHAPES) == 13 and len(set(W.SWEEP_SHAPES)) == 13
    for n, d, k in W.SWEEP_SHAPES:
        assert n in (65536, 262144, 1048576) and d in (64, 128, 256) and k in (512, 4096, 16384)
