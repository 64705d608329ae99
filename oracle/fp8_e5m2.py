"""OCP E5M2 codec in plain numpy — test infrastructure only.

The pages name a cache dtype and per-tensor ``k_scale``/``v_scale`` for the
slot-mapped write ("How PagedAttention Works in vLLM ...", section
"write_to_paged_cache: Direct In-Place Updates") but no fp8 format.  The
second 8-bit format taken here is the OCP 8-bit floating point
specification's E5M2 (``torch.float8_e5m2``):

* 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits;
* exponent field 0 is subnormal: value = m * 2**-16;
* exponent fields 1..30: value = (1 + m/4) * 2**(e - 15), so the largest
  finite magnitude is 1.75 * 2**15 = 57344;
* exponent field 31 holds infinity (m = 0) and NaN (m != 0), as in IEEE.

Encoding rounds to nearest, ties to even.  Reading: unlike the E4M3 cache
(no infinity, so it saturates), E5M2 keeps IEEE overflow: a magnitude that
rounds past 57344 -- from 61440, the midpoint to the next power of two, on
-- becomes infinity; NaN maps to the NaN code S.11111.11 with its sign.  All
arithmetic is exact in float64.
"""

import numpy as np

E5M2_MAX = 57344.0
_MIN_NORMAL_EXP = -14  # exponent field 1
_MAX_FIELD = 30        # largest finite exponent field


def e5m2_decode(codes):
    """Decode uint8 E5M2 codes to float64 (+-inf and NaN as in IEEE)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    sub = m * 2.0 ** -16
    norm = (1.0 + m / 4.0) * np.ldexp(1.0, e - 15)
    mag = np.where(e == 0, sub, norm)
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def e5m2_encode(values):
    """Encode float values (taken as given, float64) to uint8 E5M2 codes.

    Round to nearest even; overflow to +-inf; NaN -> 0x7F / 0xFF.
    """
    x = np.asarray(values, dtype=np.float64)
    neg = np.signbit(x)
    nan = np.isnan(x)
    a = np.abs(np.where(nan, 0.0, x))
    inf = np.isinf(a)
    a = np.where(inf, 1.0, a)

    # Subnormal range (below 2**-14): the uniform grid of step 2**-16; a
    # count of 4 is the smallest normal, whose code (e=1, m=0) is 4.
    small = a < 2.0 ** _MIN_NORMAL_EXP
    n_sub = np.rint(np.where(small, a, 0.0) * 2.0 ** 16).astype(np.int64)

    # Normal range: a = f * 2**k with f in [1, 2).
    f, k = np.frexp(np.where(small, 1.0, a))
    k = k - 1
    f = f * 2.0
    m = np.rint((f - 1.0) * 4.0)                    # 0..4, half-to-even
    carry = m == 4
    m = np.where(carry, 0, m).astype(np.int64)
    k = np.where(carry, k + 1, k)
    e_field = k + 15
    over = e_field > _MAX_FIELD
    norm_code = np.where(over, 0x7C, (e_field << 2) | m)

    out = np.where(small, n_sub, norm_code)
    out = np.where(inf, 0x7C, out)
    out = np.where(nan, 0x7F, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)
