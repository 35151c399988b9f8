"""Pins for the oracle's number formats and its Philox generator (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import fp, philox


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                      # finite patterns only
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(fp.bf16_bits_to_f64(bits), want)


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 1.0, 3.0, 1e5, 1e30])
def test_bf16_rne_matches_torch_on_float32_values(scale):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * scale).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(fp.f64_to_bf16_bits(x.astype(np.float64)), want)


def test_bf16_rne_ties_and_single_rounding():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties go to the even significand (1.0)
    assert fp.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 (odd) and 1+2^-6 (even)
    assert fp.f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a midpoint rounds up; a float32 detour would drop 2^-30 and tie to even
    assert fp.f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert fp.f64_to_bf16_bits(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    assert fp.f64_to_bf16_bits(0.0) == 0x0000
    # largest finite bf16 and overflow to infinity
    assert fp.f64_to_bf16_bits(3.3895313892515355e38) == 0x7F7F
    assert fp.f64_to_bf16_bits(3.5e38) == 0x7F80


def test_philox_scalar_matches_numpy():
    rng = np.random.default_rng(2)
    for _ in range(20):
        key = [int(v) for v in rng.integers(0, 2 ** 63, size=2, dtype=np.int64)]
        ctr = [int(v) for v in rng.integers(0, 2 ** 63, size=4, dtype=np.int64)]
        bg = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
        raw = [int(v) for v in bg.random_raw(8)]
        # NumPy advances the counter before producing a block
        c1 = [ctr[0] + 1] + ctr[1:]
        c2 = [ctr[0] + 2] + ctr[1:]
        assert philox.philox4x64_10(c1, key) == raw[:4]
        assert philox.philox4x64_10(c2, key) == raw[4:]


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 2 ** 40, size=64, dtype=np.int64)
    for seed, off, purpose, row in [(1, 0, 0, 0), (2 ** 62 + 5, 17, 4, 63), (5004, 3, 6, 12345)]:
        vec = philox.uniforms(seed, off, purpose, row, idx)
        ref = [philox.uniform(seed, off, purpose, row, int(i)) for i in idx]
        np.testing.assert_array_equal(vec, np.array(ref))


def test_uniform_mapping_is_open_and_float32_exact():
    assert philox.word_to_uniform(0) == 2.0 ** -24
    assert philox.word_to_uniform((1 << 64) - 1) == 1.0 - 2.0 ** -24
    u = philox.uniforms(7, 0, 1, 0, np.arange(4096))
    assert np.all((u > 0) & (u < 1))
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    # roughly uniform: mean and variance of 4096 draws
    assert abs(u.mean() - 0.5) < 0.02 and abs(u.var() - 1 / 12) < 0.01
