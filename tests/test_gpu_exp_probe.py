"""Exhaustive probe of the device exp2 (needs an MI355X).

Every decay factor of the forward kernels is exp2 of a sum of non-positive
log2-decays, and the mask is held in [0, 1] and non-increasing away from the
diagonal (page "GPU Hierarchy Meets Structured Matrices", abstract: a stable
segsum without monotonicity violations) only if that exp2 is itself monotone
and at most 1 on non-positive arguments.  The probe evaluates it on every
fp32 value in [-160, 0] (about 1.1e9 of them; below -150 every result is 0),
and then on every non-positive fp32 down to -inf, on the device, counting
increases as the argument decreases, results above 1 and results below 0 or
NaN."""
import pytest

pytestmark = pytest.mark.gpu

MINUS_ZERO = 0x80000000
MINUS_160 = 0xC3200000
MINUS_INF = 0xFF800000


def test_exp2_monotone_and_at_most_one_on_minus_160_to_0():
    import ssd_chunked_scan_amd as ssd
    r = ssd.ssd_debug_exp2_probe(MINUS_ZERO, MINUS_160 - MINUS_ZERO + 1)
    print("exp2 on [-160, 0]:", r)
    assert r == {"increases": 0, "above_one": 0, "negative_or_nan": 0}


def test_exp2_monotone_on_every_non_positive_float():
    import ssd_chunked_scan_amd as ssd
    r = ssd.ssd_debug_exp2_probe(MINUS_ZERO, MINUS_INF - MINUS_ZERO + 1)
    print("exp2 on [-inf, 0]:", r)
    assert r == {"increases": 0, "above_one": 0, "negative_or_nan": 0}


def test_probe_range_checks_and_denormal_arguments():
    """Positive arguments are refused (the probe covers non-positive ones
    only); the first 2^20 patterns from -0 (-0 and negative denormals, whose
    exp2 is 1 within rounding) never exceed 1."""
    import ssd_chunked_scan_amd as ssd
    with pytest.raises(ssd.SsdError):
        ssd.ssd_debug_exp2_probe(0x00000000, 16)
    r = ssd.ssd_debug_exp2_probe(MINUS_ZERO, 1 << 20)
    assert r["above_one"] == 0 and r["negative_or_nan"] == 0
