"""Pins of how operand values reach both sides: the oracle's widening of bf16 bit
patterns to fp64, and the seeded generator's fp32 -> bf16 rounding, each against
torch's own bfloat16 conversions (an implementation that shares nothing with
either)."""
import numpy as np
import pytest
import torch

import oracle
from synth import f32_to_bf16_bits
from synth.inputs import bf16_bits_to_f32

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_widen_bf16_every_bit_pattern():
    """All 65536 bf16 patterns: the same fp64 value as torch's conversion,
    including signed zeros, subnormals and infinities; NaN patterns stay NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "bf16")
    exp = _torch_bf16_to_f64(bits)
    nan = np.isnan(exp)
    assert nan.sum() == 2 * 127                      # exponent all ones, mantissa != 0
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], exp[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(exp[~nan]))
    # a few fixed points worked by hand: 0x3F80 = 1, 0xC000 = -2, 0x0001 = 2^-133
    assert oracle.widen(np.array([0x3F80, 0xC000, 0x0001], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, 2.0 ** -133]


def test_widen_fp32_and_fp64_are_value_for_value():
    g = np.random.default_rng(0)
    x = g.standard_normal(1000).astype(np.float32)
    np.testing.assert_array_equal(oracle.widen(x, "f32"), x.astype(np.float64))
    x64 = g.standard_normal(10)
    np.testing.assert_array_equal(oracle.widen(x64, "f64"), x64)


def _torch_round(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_rounding_matches_torch():
    """Round to nearest, ties to even, against torch's fp32 -> bf16 cast: random
    values over the whole exponent range, exact ties on even and odd
    significands, just-above and just-below ties, subnormals, the largest finite
    values (which round to infinity), infinities and signed zeros."""
    g = np.random.default_rng(1)
    rnd = g.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    specials = []
    for hi in (0x3F80, 0x3F81, 0x0001, 0x0002, 0x007F, 0x7F7F, 0x7F7E, 0xBF80, 0xBF81, 0x8001):
        for lo in (0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            specials.append((hi << 16) | lo)
    specials += [0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001, 0x007FFFFF]
    u = np.concatenate([rnd, np.array(specials, np.uint32)])
    x = u.view(np.float32)
    finite = ~np.isnan(x)
    got, exp = f32_to_bf16_bits(x), _torch_round(x)
    np.testing.assert_array_equal(got[finite], exp[finite])
    # NaN inputs give a NaN pattern (torch's and ours are both quiet NaNs)
    assert np.all(np.isnan(bf16_bits_to_f32(got[~finite])))
    # ties, by hand: 1 + 2^-8 (0x3F808000) lies halfway between 1 (0x3F80, even) and
    # 1 + 2^-7 (0x3F81): it goes to the even 0x3F80; 0x3F818000 goes up to 0x3F82
    ties = np.array([0x3F808000, 0x3F818000], np.uint32).view(np.float32)
    assert f32_to_bf16_bits(ties).tolist() == [0x3F80, 0x3F82]


def test_bf16_bits_to_f32_inverts_the_rounding_on_representable_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    ok = ~np.isnan(f)
    np.testing.assert_array_equal(f32_to_bf16_bits(f[ok]), bits[ok])
