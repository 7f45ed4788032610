"""The seeded input generator: deterministic, random access, N(0,1), bf16 RNE."""
import numpy as np

import fixtures


def test_deterministic_and_random_access():
    a = fixtures.normal_bf16(7, 1, (3, 1000))
    b = fixtures.normal_bf16(7, 1, (3, 1000))
    assert np.array_equal(a, b)
    flat = a.reshape(-1)
    assert np.array_equal(fixtures.normal_bf16(7, 1, (501,), offset=999), flat[999:1500])
    rows = fixtures.rows_bf16(7, 1, [2, 0], 1000)
    assert np.array_equal(rows, a[[2, 0]])
    assert not np.array_equal(a, fixtures.normal_bf16(7, 2, (3, 1000)))
    assert not np.array_equal(a, fixtures.normal_bf16(8, 1, (3, 1000)))


def test_standard_normal_moments():
    z = fixtures.normal_f64(3, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(np.mean(z ** 4) - 3) < 0.05          # Gaussian kurtosis
    assert abs(np.mean(np.abs(z) < 1.0) - 0.6827) < 0.01


def test_bf16_rounding_is_nearest_even():
    z = fixtures.normal_f64(5, 2, 20000)
    bits = fixtures.normal_bf16(5, 2, (20000,))
    got = fixtures.bf16_to_f64(bits)
    f = z.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lo = (u >> 16) << 16
    hi = lo + (1 << 16)
    flo = lo.astype(np.uint32).view(np.float32).astype(np.float64)
    fhi = hi.astype(np.uint32).view(np.float32).astype(np.float64)
    fd = f.astype(np.float64)
    dlo, dhi = np.abs(fd - flo), np.abs(fhi - fd)
    want = np.where(dlo < dhi, flo, np.where(dhi < dlo, fhi,
                    np.where(((lo >> 16) & 1) == 0, flo, fhi)))
    assert np.array_equal(got, want)
