"""The single-pass MFMA kernel computes floor(a / waves) for its slice
rotation and bounds through a float reciprocal: floor((a + 0.5) * rcp(waves))
for 0 <= a <= 65536 and 1 <= waves <= 16.  This pins the claim on the CPU
with float32 arithmetic and a reciprocal off by up to one ulp either way
(the hardware reciprocal's error bound), against exact integer division."""
import numpy as np


def test_reciprocal_floor_division_is_exact():
    a = np.arange(0, 65537, dtype=np.int64)
    af = a.astype(np.float32)
    for waves in range(1, 17):
        r = np.float32(1.0) / np.float32(waves)
        for rr in (np.nextafter(r, np.float32(0)), r, np.nextafter(r, np.float32(1))):
            q = ((af + np.float32(0.5)) * rr).astype(np.float32)  # one fp32 product
            got = np.floor(q).astype(np.int64)
            assert np.array_equal(got, a // waves), f"waves={waves}"


def test_margin_is_what_makes_it_exact():
    # without the half step, an exact multiple times a reciprocal rounded
    # down lands just below the integer: the plain form fails somewhere
    a = np.arange(0, 65537, dtype=np.int64).astype(np.float32)
    bad = 0
    for waves in (3, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15):
        r = np.nextafter(np.float32(1.0) / np.float32(waves), np.float32(0))
        got = np.floor((a * r).astype(np.float32)).astype(np.int64)
        bad += int(np.sum(got != np.arange(0, 65537) // waves))
    assert bad > 0
