"""OCP E4M3 ("fn") codec in plain numpy — test infrastructure only.

The pages name a cache dtype and per-tensor ``k_scale``/``v_scale`` for the
slot-mapped write ("How PagedAttention Works in vLLM ...", section
"write_to_paged_cache: Direct In-Place Updates") but not the fp8 format.
Reading taken here: the OCP 8-bit floating point specification's E4M3 format
as used by ``torch.float8_e4m3fn``:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 is subnormal: value = m * 2**-9;
* otherwise value = (1 + m/8) * 2**(e - 7);
* no infinities; S.1111.111 is NaN, so the largest finite magnitude is
  S.1111.110 = 448.

Encoding (the cache write for an fp8 cache) rounds to nearest, ties to
even, and saturates finite values beyond the largest magnitude to +-448;
NaN maps to the NaN code with its sign.  All arithmetic below is exact in
float64: inputs are float32 values, and scaling by powers of two and
rounding to an integer lose nothing.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6   # exponent field 1
_MAX_EXP = 8           # exponent field 15


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** -9
    norm = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(values):
    """Encode float values (taken as given, float64) to uint8 E4M3 codes.

    Round to nearest even; saturate to +-448; NaN -> 0x7F / 0xFF.
    """
    x = np.asarray(values, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    # infinities saturate like any other out-of-range magnitude
    a = np.where(np.isinf(a), 2.0 ** 20, a)

    out = np.zeros(x.shape, dtype=np.int64)

    # Subnormal range (below the smallest normal 2**-6): quantise on the
    # uniform grid of step 2**-9.  A result of 8 steps is the smallest
    # normal, whose code (e=1, m=0) is exactly 8, so the code is the count.
    small = a < 2.0 ** _MIN_NORMAL_EXP
    n_sub = np.rint(np.where(small, a, 0.0) * 2.0 ** 9)   # half-to-even
    out = np.where(small, n_sub.astype(np.int64), out)

    # Normal range: a = f * 2**k with f in [1, 2).
    f, k = np.frexp(np.where(small, 1.0, a))        # f in [0.5, 1)
    k = k - 1
    f = f * 2.0                                     # [1, 2)
    m = np.rint((f - 1.0) * 8.0)                    # 0..8, half-to-even
    carry = m == 8
    m = np.where(carry, 0, m).astype(np.int64)
    k = np.where(carry, k + 1, k)
    overflow = (k > _MAX_EXP) | ((k == _MAX_EXP) & (m > 6))
    e_field = k + 7
    norm_code = (e_field << 3) | m
    norm_code = np.where(overflow, 0x7E, norm_code)
    out = np.where(small, out, norm_code)

    out = np.where(nan, 0x7F, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)
