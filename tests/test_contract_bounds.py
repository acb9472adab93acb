"""CPU pins of the precision statements the C ABI makes about its two FFN contracts.

The FP32 contract hands h = silu(g) * u to the down projection as two bf16 terms,
h_hi = bf16(h) and h_lo = bf16(h - h_hi), both rounded to nearest even.  The header
states that h_hi + h_lo is within 2^-16 * |h| of h (plus half the smallest bf16
subnormal for tiny h).  This checks that bound over a million fp32 values of every
binade the activations can take, plus the rounding corners, with the rounding written
here from its definition (not taken from the library or the oracle).
"""
import numpy as np

from fractions import Fraction


def bf16_rne(f: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values; finite inputs."""
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF0000
    rem = u & 0xFFFF
    odd = (lower >> 16) & 1
    up = (rem > 0x8000) | ((rem == 0x8000) & (odd == 1))
    return (lower + np.where(up, 0x10000, 0)).astype(np.uint32).view(np.float32)


def split(h: np.ndarray):
    h = np.asarray(h, np.float32)
    hi = bf16_rne(h)
    lo = bf16_rne((h - hi).astype(np.float32))  # h - hi is exact in fp32 (the two share the leading bits)
    return hi, lo


def test_bf16_rounding_helper_is_nearest_even():
    # exact ties and near-ties, checked against exact rational distances
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -3.0078125 - 2 ** -10,
                     65504.0, 1e-30, -7.25e12], np.float32)
    got = bf16_rne(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        u = int(np.array([v], np.float32).view(np.uint32)[0]) & 0xFFFF0000
        cands = [np.array([c], np.uint32).view(np.float32)[0].item() for c in (u, u + 0x10000)]
        d = [abs(Fraction(c) - Fraction(v)) for c in cands]
        if d[0] != d[1]:
            assert g == cands[int(d[1] < d[0])]
        else:
            assert g == cands[0] if ((u >> 16) & 1) == 0 else g == cands[1]


def test_h_split_error_bound():
    rng = np.random.default_rng(2024)
    n = 1 << 20
    # every fp32 bit pattern with exponents from 2^-120 to 2^60, random significands and signs
    exps = rng.integers(127 - 120, 127 + 60, n).astype(np.uint32)
    sig = rng.integers(0, 1 << 23, n).astype(np.uint32)
    sign = rng.integers(0, 2, n).astype(np.uint32)
    h = ((sign << 31) | (exps << 23) | sig).view(np.float32)
    # the rounding corners: significands just below, at and above the bf16 halfway points
    corners = np.array([0x3F808000, 0x3F807FFF, 0x3F808001, 0x3F818000, 0x3F7FFFFF, 0x3F7F8000, 0xBF7FC000,
                        0x00800000, 0x00FFFFFF, 0x5F7FFFFF], np.uint32).view(np.float32)
    h = np.concatenate([h, corners])
    hi, lo = split(h)
    err = np.abs(h.astype(np.float64) - (hi.astype(np.float64) + lo.astype(np.float64)))
    bound = 2.0 ** -16 * np.abs(h.astype(np.float64)) + 2.0 ** -134
    worst = float(np.max(err / bound))
    assert worst <= 1.0, worst
    # and the bound is not loose by orders of magnitude: the split is ~17 bits, not 24
    assert float(np.max(err / np.abs(h.astype(np.float64)))) > 2.0 ** -19
