"""The exact three-way bf16 split of an fp32 router weight (host-side check of the arithmetic fact the matrix-core
router relies on; Routing Mamba landing page (chapterpal.com), Knowl 1: the router logits are x_t W_r in fp32).

With hi = bf16(w), mid = bf16(w - hi) and lo = w - hi - mid, both differences are exact in fp32 and lo has at most
8 significant bits, so w = hi + mid + lo exactly and every product of a bf16 x with a part is exact in fp32. The
test draws fp32 values over the normal exponent range (plus binade edges and values that round up into the next
binade) and checks each claim in float64 arithmetic, which holds every such sum and product exactly.
"""
import numpy as np


def _bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest, ties to even) -> fp32, on the bit pattern (finite inputs)."""
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _sig_bits(a: np.ndarray) -> np.ndarray:
    """Significant bits of each finite fp32 value (0 for zero): bit span of its integer significand."""
    out = np.zeros(a.shape, np.int64)
    nz = a != 0
    m, e = np.frexp(a[nz].astype(np.float64))  # a = m * 2**e, 0.5 <= |m| < 1
    ints = np.abs(np.ldexp(m, 53)).astype(np.uint64)  # significand scaled to an integer
    tz = np.zeros(ints.shape, np.int64)
    t = ints.copy()
    for _ in range(64):  # count trailing zeros
        z = (t & 1) == 0
        if not np.any(z & (t != 0)):
            break
        tz += (z & (t != 0))
        t = np.where(z & (t != 0), t >> 1, t)
    out[nz] = 53 - tz
    return out


def _values(rng: np.random.Generator, n: int) -> np.ndarray:
    mant = rng.integers(0, 1 << 23, n, dtype=np.int64)
    expo = rng.integers(1 + 16, 255 - 1, n, dtype=np.int64)  # normal values whose residuals stay normal
    sign = rng.integers(0, 2, n, dtype=np.int64)
    bits = (sign << 31) | (expo << 23) | mant
    w = bits.astype(np.uint32).view(np.float32)
    edges = np.array([1.0, -1.0, 1.0 + 2.0 ** -23, 2.0 - 2.0 ** -23, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9,
                      np.float32(1.9960938), np.float32(0.03125) * (1 + 2.0 ** -20), np.float32(3.0e38),
                      np.float32(-2.5e-34)], np.float32)
    return np.concatenate([w, edges, rng.normal(0, 1.0 / 32.0, n).astype(np.float32)])


def test_three_bf16_parts_sum_to_the_fp32_weight_exactly():
    rng = np.random.default_rng(2026)
    w = _values(rng, 200_000)
    hi = _bf16_rne(w)
    r1 = (w - hi).astype(np.float32)
    mid = _bf16_rne(r1)
    r2 = (r1 - mid).astype(np.float32)
    lo = _bf16_rne(r2)
    # the two fp32 differences are exact
    assert np.all(r1.astype(np.float64) == w.astype(np.float64) - hi.astype(np.float64))
    assert np.all(r2.astype(np.float64) == r1.astype(np.float64) - mid.astype(np.float64))
    # the remainder has at most 8 significant bits, so bf16 holds it
    assert np.all(_sig_bits(r2) <= 8)
    assert np.all(lo == r2)
    # hence the parts sum to w exactly
    assert np.all(hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64) == w.astype(np.float64))


def test_products_of_bf16_rows_with_the_parts_are_exact_in_fp32():
    rng = np.random.default_rng(7)
    w = rng.normal(0, 1.0 / 32.0, 50_000).astype(np.float32)
    x = _bf16_rne(rng.normal(0, 1.0, 50_000).astype(np.float32))
    hi = _bf16_rne(w)
    mid = _bf16_rne((w - hi).astype(np.float32))
    lo = _bf16_rne((w - hi - mid).astype(np.float32))
    for part in (hi, mid, lo):
        p64 = x.astype(np.float64) * part.astype(np.float64)
        assert np.all(p64.astype(np.float32).astype(np.float64) == p64)  # representable in fp32
        assert np.all(_sig_bits(p64.astype(np.float32)) <= 16)
    # and x * w equals the sum of the three exact products
    total = sum(x.astype(np.float64) * p.astype(np.float64) for p in (hi, mid, lo))
    assert np.all(total == x.astype(np.float64) * w.astype(np.float64))


def test_split_mutant_without_the_middle_part_is_not_exact():
    """A two-part split (hi + bf16(w - hi)) loses bits: the check above must be able to fail."""
    rng = np.random.default_rng(11)
    w = _values(rng, 10_000)
    hi = _bf16_rne(w)
    lo = _bf16_rne((w - hi).astype(np.float32))
    assert np.any(hi.astype(np.float64) + lo.astype(np.float64) != w.astype(np.float64))
