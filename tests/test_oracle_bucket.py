"""Pins for the oracle's relative-position bucket (CPU only).

The oracle decides the ceiling with exact integers. These tests tie it to
facts that do not come from its own code: the identity region, odd
symmetry, monotonicity, where the top bucket is reached, the closed form at
|r| = M-1, hand-evaluated points, the full coverage of the log range, and a
high-precision decimal evaluation of the real-valued formula.
"""

import decimal
import math

import numpy as np
import pytest

from oracle import bucket

CONFIG_PARAMS = [(256, 512), (8, 20), (16, 64), (32, 129), (4, 7), (2, 9)]


@pytest.mark.parametrize("P,M", CONFIG_PARAMS)
def test_identity_region_and_symmetry(P, M):
    mid = P // 2
    for r in range(-mid, mid + 1):
        assert bucket.log_bucket(r, P, M) == r
    for r in range(0, 3 * M):
        assert bucket.log_bucket(-r, P, M) == -bucket.log_bucket(r, P, M)


@pytest.mark.parametrize("P,M", CONFIG_PARAMS)
def test_monotone_and_top_at_m_minus_1(P, M):
    vals = [bucket.log_bucket(r, P, M) for r in range(-4 * M, 4 * M + 1)]
    assert all(a <= b for a, b in zip(vals, vals[1:]))
    mid = P // 2
    # at |r| = M-1 the real argument is exactly mid-1, so b = 2*mid - 1
    assert bucket.log_bucket(M - 1, P, M) == 2 * mid - 1
    assert bucket.log_bucket(-(M - 1), P, M) == -(2 * mid - 1)


@pytest.mark.parametrize("P,M", [(256, 512), (16, 64), (8, 20)])
def test_log_range_covers_every_bucket_once_in_order(P, M):
    """On mid < r <= M-1 the ceiling climbs from 1 to mid-1 in steps of at
    most 1 (the slope (mid-1)/(r ln((M-1)/mid)) stays below 1 there for
    these parameters), so every bucket mid+1 .. 2mid-1 appears."""
    mid = P // 2
    got = sorted({bucket.log_bucket(r, P, M) for r in range(mid + 1, M)})
    assert got == list(range(mid + 1, 2 * mid))


def test_hand_evaluated_points_256_512():
    # mid = 128, ln(511/128) = 1.3843823...; x = 127 ln(r/128) / 1.3843823
    # r=129: x = 127*0.0077821/1.3843823 = 0.714  -> 128 + 1   = 129
    # r=200: x = 127*0.4462871/1.3843823 = 40.94  -> 128 + 41  = 169
    # r=256: x = 127*0.6931472/1.3843823 = 63.59  -> 128 + 64  = 192
    # r=400: x = 127*1.1394343/1.3843823 = 104.53 -> 128 + 105 = 233
    # r=511: x = 127 exactly                      -> 128 + 127 = 255
    # r=512: x = 127*1.3862944/1.3843823 = 127.18 -> 128 + 128 = 256
    # r=8191: x = 127*4.1587659/1.3843823 = 381.5 -> 128 + 382 = 510
    expect = {129: 129, 200: 169, 256: 192, 400: 233, 511: 255, 512: 256, 8191: 510}
    for r, b in expect.items():
        assert bucket.log_bucket(r, 256, 512) == b
        assert bucket.log_bucket(-r, 256, 512) == -b


def test_table_clamp_and_saturation_256_512():
    """Rows are clamp(b + 256, 0, 511): the top row is first reached at
    r = 506 (b = 255), the bottom row at r = -512 (b = -256)."""
    T = bucket.rel_index_table(8192, 256, 512)
    off = 8191
    assert T.shape == (16383,)
    assert T.min() == 0 and T.max() == 511
    assert T[off + 0] == 256
    assert T[off + 505] < 511 and T[off + 506] == 511
    assert np.all(T[off + 506:] == 511)
    assert T[off - 511] == 1 and T[off - 512] == 0
    assert np.all(T[: off - 511] == 0)
    assert np.all(np.diff(T) >= 0)


def test_identity_table_c1():
    """Without bucketing and span 64: rows clamp(r + 64, 0, 127)."""
    T = bucket.rel_index_table(128, 0, 64)
    r = np.arange(-127, 128)
    assert np.array_equal(T, np.clip(r + 64, 0, 127))


def _decimal_bucket(r, P, M):
    """The real-valued formula at 60 significant digits (independent of the
    integer comparison the oracle uses)."""
    mid = P // 2
    a = abs(r)
    if a <= mid:
        return r, None
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        x = (decimal.Decimal(mid - 1) * (decimal.Decimal(a) / mid).ln()
             / (decimal.Decimal(M - 1) / mid).ln())
        n = x.to_integral_value(rounding=decimal.ROUND_CEILING)
        margin = abs(x - x.to_integral_value(rounding=decimal.ROUND_HALF_EVEN))
    b = mid + int(n)
    return (b if r > 0 else -b), margin


@pytest.mark.parametrize("P,M", [(256, 512), (16, 64), (8, 20), (64, 300)])
def test_decimal_evaluation_agrees(P, M):
    checked = 0
    for r in range(1, 2 * M + 40):
        want, margin = _decimal_bucket(r, P, M)
        got = bucket.log_bucket(r, P, M)
        if margin is not None and margin < decimal.Decimal("1e-40"):
            # the argument is an integer: both sides must give mid + x
            assert got == want or r == M - 1
            continue
        assert got == want, (r, got, want)
        checked += 1
    assert checked > M


def test_float64_margin_for_configs():
    """For 256/512 and every |r| <= 8191 the float64 evaluation agrees with
    the exact one, and apart from the exact hit at |r| = 511 the real
    argument stays at least 1e-5 from an integer."""
    mid, M = 128, 512
    c = math.log((M - 1) / mid)
    worst = 1.0
    for r in range(mid + 1, 8192):
        x = (mid - 1) * math.log(r / mid) / c
        if r == M - 1:
            continue
        worst = min(worst, abs(x - round(x)))
        assert mid + math.ceil(x) == bucket.log_bucket(r, 256, 512)
    assert worst > 1e-5


def test_parameter_checks():
    with pytest.raises(ValueError):
        bucket.log_bucket(5, 1, 512)      # mid = 0
    with pytest.raises(ValueError):
        bucket.log_bucket(5, 256, 129)    # M - 1 <= mid
    with pytest.raises(ValueError):
        bucket.rel_index_table(0, 256, 512)
