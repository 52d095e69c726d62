"""Relative-position bucket, computed with exact integer arithmetic.

TEST INFRASTRUCTURE: only tests, the smoke entry and the benchmark's CPU
baseline may import this module. The product path never does.

Source. The DisentangledFlash README ("Status") names the method as
DeBERTa-v2/v3 C2P/P2C disentangled attention, and its "Attribution" section
says the auditable reference path derives from the DeBERTa-v2/v3 modeling
code of Hugging Face Transformers. None of the pages prints the bucket
function; what is written here is the DeBERTa-v2 log-bucket mapping restated
as mathematics:

    mid = floor(P / 2)
    b(r) = r                                             if |r| <= mid
    b(r) = sign(r) * (mid + ceil((mid-1) * ln(|r|/mid) / ln((M-1)/mid)))
                                                         otherwise
    span s = P; the row used for distance r is clamp(b(r) + s, 0, 2s - 1).

With P <= 0 there is no bucketing: b(r) = r and s = M.

The ceiling is taken of the real number, decided without any logarithm:
for |r| > mid, ceil(x) is the least integer k with
    (M-1)^k * mid^(mid-1) >= |r|^(mid-1) * mid^k,
which is the integer form of  k >= (mid-1) ln(|r|/mid) / ln((M-1)/mid)
(valid because ln((M-1)/mid) > 0, which the parameter check demands).
"""

from __future__ import annotations

import functools
import math

import numpy as np


def span(position_buckets: int, max_relative_positions: int) -> int:
    """Number of relative rows on each side: P when bucketing, else M."""
    return position_buckets if position_buckets > 0 else max_relative_positions


def check_params(position_buckets: int, max_relative_positions: int) -> None:
    """Parameters for which the bucket is defined (raises ValueError)."""
    P, M = position_buckets, max_relative_positions
    if P > 0:
        mid = P // 2
        if mid < 1:
            raise ValueError("position_buckets must be >= 2 when bucketing")
        if M - 1 <= mid:
            raise ValueError("max_relative_positions - 1 must exceed position_buckets // 2")
    else:
        if M < 1:
            raise ValueError("max_relative_positions must be >= 1 without bucketing")


def _ceil_log_ratio(a: int, mid: int, M: int) -> int:
    """ceil((mid-1) * ln(a/mid) / ln((M-1)/mid)) for integer a > mid, exactly."""
    e = mid - 1
    if e == 0:
        return 0
    lhs_const = mid ** e          # mid^(mid-1)
    rhs_const = a ** e            # a^(mid-1)

    def ok(k: int) -> bool:      # (M-1)^k * mid^(mid-1) >= a^(mid-1) * mid^k
        return (M - 1) ** k * lhs_const >= rhs_const * mid ** k

    # start from a floating estimate and walk to the exact answer
    k = max(0, int(math.ceil(e * math.log(a / mid) / math.log((M - 1) / mid))))
    while k > 0 and ok(k - 1):
        k -= 1
    while not ok(k):
        k += 1
    return k


@functools.lru_cache(maxsize=None)
def _bucket_cached(r: int, P: int, M: int) -> int:
    if P <= 0:
        return r
    mid = P // 2
    a = abs(r)
    if a <= mid:
        return r
    k = _ceil_log_ratio(a, mid, M)
    return (mid + k) if r > 0 else -(mid + k)


def log_bucket(r: int, position_buckets: int, max_relative_positions: int) -> int:
    """b(r) for one signed relative distance r (query position minus key
    position for the content-to-position term)."""
    check_params(position_buckets, max_relative_positions)
    return _bucket_cached(int(r), int(position_buckets), int(max_relative_positions))


def rel_index_table(max_len: int, position_buckets: int,
                    max_relative_positions: int) -> np.ndarray:
    """T[r + max_len - 1] = clamp(b(r) + s, 0, 2s - 1) for
    r in [-(max_len-1), max_len-1]; int64 array of 2*max_len - 1 entries."""
    check_params(position_buckets, max_relative_positions)
    if max_len < 1:
        raise ValueError("max_len must be >= 1")
    s = span(position_buckets, max_relative_positions)
    out = np.empty(2 * max_len - 1, dtype=np.int64)
    for idx in range(2 * max_len - 1):
        r = idx - (max_len - 1)
        b = _bucket_cached(r, int(position_buckets), int(max_relative_positions))
        out[idx] = min(max(b + s, 0), 2 * s - 1)
    return out
