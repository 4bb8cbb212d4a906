"""The exactness argument behind the counts x grad_out product on bfloat16
matrix cores (the compensated split of the FBTriton page's histogram-reuse
backward, "Fusion boundaries", taken in its exact form), checked on the
host with numpy, independently of the kernels:

- an fp32 value x of magnitude at least 2^-100 (so that every part is a
  normal number) is the exact sum of three bfloat16 values: hi = x with
  the low 16 bits cleared, mid = the same of x - hi, lo = x - hi - mid
  (each difference exact in fp32), and lo has its low 16 bits zero, so it
  is a bfloat16 value too; for smaller x the lo part can be subnormal and
  its truncation to bfloat16 drops less than 2^-133;
- a count of at most 8 significant bits (any integer up to 255, and every
  8-bit part c & (0xff << 8k) of a wider count) is exact in bfloat16, and
  its product with any bfloat16 value is exact in fp32 (16 significant
  bits at most), so the three products add up to count * x with only the
  additions rounding."""
import numpy as np


def _bf16_trunc(x):
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _split3(x):
    x = x.astype(np.float32)
    hi = _bf16_trunc(x)
    r1 = (x - hi).astype(np.float32)
    mid = _bf16_trunc(r1)
    lo = (r1 - mid).astype(np.float32)
    return hi, mid, lo


def _is_bf16(v):
    return np.all((v.view(np.uint32) & np.uint32(0xFFFF)) == 0)


def _samples():
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-30, 30, 100_000)).astype(np.float32),
        rng.integers(0, 2**32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1.1754944e-38, 1.0 + 2.0 ** -23,
                  np.float32(np.pi), 65504.0, 2.0 ** -126], np.float32),
    ]
    x = np.concatenate(parts)
    return x[np.isfinite(x)]


def test_three_bf16_parts_sum_exactly():
    x = _samples()
    x = x[(np.abs(x) >= 2.0 ** -100) | (x == 0)]
    hi, mid, lo = _split3(x)
    for part in (hi, mid, lo):
        assert _is_bf16(part)
    # the sum in float64 (exact for three floats of these magnitudes) is x
    s = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert np.array_equal(s, x.astype(np.float64))


def test_tiny_values_lose_less_than_two_to_minus_133():
    x = _samples()
    x = np.concatenate([x[np.abs(x) < 2.0 ** -100],
                        np.array([2.0 ** -110, 3.0 * 2.0 ** -120, 2.0 ** -126, 2.0 ** -140],
                                 np.float32)])
    assert x.size > 1000
    hi, mid, lo = _split3(x)
    lo_t = _bf16_trunc(lo)  # the bfloat16 the kernel packs
    s = hi.astype(np.float64) + mid.astype(np.float64) + lo_t.astype(np.float64)
    assert np.max(np.abs(s - x.astype(np.float64))) < 2.0 ** -133


def test_eight_bit_counts_times_parts_are_exact_products():
    x = _samples()[:50_000]
    x = x[np.abs(x) < 1e30]  # products stay finite
    hi, mid, lo = _split3(x)
    for c in (1, 2, 3, 17, 128, 255):
        cf = np.float32(c)
        assert _is_bf16(np.array([cf], np.float32))
        for part in (hi, mid, lo):
            prod32 = (cf * part).astype(np.float32)
            assert np.array_equal(prod32.astype(np.float64), c * part.astype(np.float64))
        total = (cf * hi).astype(np.float64) + (cf * mid) + (cf * lo)
        assert np.array_equal(total, c * x.astype(np.float64))


def test_wide_counts_cut_into_exact_eight_bit_parts():
    rng = np.random.default_rng(11)
    counts = np.concatenate([rng.integers(0, 2**32, 10_000, dtype=np.uint64),
                             np.array([0, 255, 256, 257, 65535, 65536, 2**24 + 1, 2**32 - 1])])
    counts = counts.astype(np.uint32)
    parts = [(counts & np.uint32(0xFF << (8 * k))).astype(np.float32) for k in range(4)]
    for p in parts:
        assert _is_bf16(p)
    assert np.array_equal(sum(p.astype(np.float64) for p in parts), counts.astype(np.float64))
