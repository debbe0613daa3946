"""Host-side checks of numerical identities the HIP kernels rely on (no GPU needed)."""
import numpy as np

from oracle import fp8_e4m3 as F8


def _quotient_via_f64_reciprocal(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    return (x.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def test_quotient_through_fp64_reciprocal_is_correctly_rounded():
    """The block quantisers form fl32(x / s) as fl32(fl64(x) * fl64(1 / s)).

    A quotient of two fp32 values is never an fp32 rounding midpoint and lies more than
    2^-49 (relative) from every one, while the fp64 product is within 2^-52 of the exact
    quotient, so the two roundings agree.  numpy's float32 division is the IEEE reference.
    """
    rng = np.random.default_rng(5)
    n = 1_000_000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    amax = (np.abs(rng.standard_normal(n)) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    assert np.array_equal(_quotient_via_f64_reciprocal(x, s), (x / s).astype(np.float32))


def test_quotient_near_e4m3_rounding_midpoints():
    """Values built to land next to the e4m3 rounding midpoints after the division, where a
    quotient off by one fp32 ulp would change the code."""
    rng = np.random.default_rng(6)
    vals = F8.decode(np.arange(256, dtype=np.uint8))
    vals = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (vals[:-1] + vals[1:]) / 2.0
    s = (np.abs(rng.standard_normal(4096)) * np.exp2(rng.integers(-8, 8, 4096)) / 448.0).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    m = np.repeat(mids, len(s))
    ss = np.tile(s, len(mids))
    x0 = (m * ss).astype(np.float32)
    for dx in (-2, -1, 0, 1, 2):   # a few fp32 steps around each target
        x = x0.copy()
        for _ in range(abs(dx)):
            x = np.nextafter(x, np.float32(np.inf) if dx > 0 else np.float32(-np.inf))
        want = (x / ss).astype(np.float32)
        got = _quotient_via_f64_reciprocal(x, ss)
        assert np.array_equal(got, want)
        assert np.array_equal(F8.encode(np.clip(got, -448, 448)), F8.encode(np.clip(want, -448, 448)))
