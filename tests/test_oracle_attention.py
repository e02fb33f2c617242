"""The oracle's attention pinned to brute force, a library routine, closed
forms and invariants (CPU only)."""

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_bf16_decode_is_exact_and_rounding_is_rne():
    # patterns decode to the float32 with the same upper half
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000], np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 3.140625
    assert vals[3] == 2.0 ** -133            # smallest bf16 subnormal
    assert np.isinf(vals[4]) and vals[4] > 0 and np.isinf(vals[5]) and vals[5] < 0
    assert vals[6] == 0.0 and np.signbit(vals[7])
    # ties go to the even pattern; values above the tie round up
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    tie_even = np.float32(one + ulp / 2)           # between 0x3F80 and 0x3F81 -> 0x3F80
    tie_odd = np.float32(one + ulp + ulp / 2)      # between 0x3F81 and 0x3F82 -> 0x3F82
    above = np.nextafter(tie_even, np.float32(2))
    got = oracle.f32_to_bf16_bits(np.array([tie_even, tie_odd, above], np.float32))
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F81]
    assert oracle.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] & 0x7F80 == 0x7F80


def test_bf16_oracle_matches_f32_oracle_on_the_same_values():
    """The same (bf16-representable) values given as f32 or as bf16 bits give
    the same float64 result: the bf16 path only changes the decoding."""
    rng = np.random.default_rng(5)
    L, hq, hkv, d, bs = 40, 4, 2, 16, 16
    nb = 4
    q32 = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32))).astype(np.float32)
    kc32 = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(rng.standard_normal((nb, hkv, d // 8, bs, 8)).astype(np.float32))).astype(np.float32)
    vc32 = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(rng.standard_normal((nb, hkv, d, bs)).astype(np.float32))).astype(np.float32)
    tab = np.array([[2, 0, 3]], np.int32)
    lens = np.array([L], np.int32)
    a = oracle.decode(q32, kc32, vc32, tab, lens, 0.25, bs, "f32")
    b = oracle.decode(oracle.f32_to_bf16_bits(q32), oracle.f32_to_bf16_bits(kc32),
                      oracle.f32_to_bf16_bits(vc32), tab, lens, 0.25, bs, "bf16")
    assert np.array_equal(a, b)


def test_decode_reads_only_the_context():
    """Only the first ceil(L/bs) table entries and the first L slots are read."""
    rng = np.random.default_rng(6)
    nb, hkv, d, bs = 6, 1, 8, 16
    kc = rng.standard_normal((nb, hkv, d // 4, bs, 4)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, d, bs)).astype(np.float32)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    tab = np.array([[4, 1, 5, 2]], np.int32)
    lens = np.array([20], np.int32)
    base = oracle.decode(q, kc, vc, tab, lens, 0.3, bs, "f32")
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[1, :, :, 4:, :] = np.nan       # tail of the second (last used) page
    vc2[1, :, :, 4:] = np.nan
    kc2[[0, 2, 3, 5]] = np.nan         # pages not in use, incl. the unused entries
    vc2[[0, 2, 3, 5]] = np.nan
    tab2 = tab.copy()
    tab2[0, 2:] = [123456, -1]         # entries past ceil(L/bs) are never read
    got = oracle.decode(q, kc2, vc2, tab2, lens, 0.3, bs, "f32")
    assert np.array_equal(base, got)
