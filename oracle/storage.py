"""Rounding of a result to the storage format of its tensor.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A parameter kept in bfloat16 holds, after a step, the step's result rounded
once to bfloat16 (the reading the tests take of a low-precision parameter:
the update is computed at full precision and the stored value is its
rounding).  bfloat16 keeps the float32 exponent range and 8 significant bits
(7 stored, one implicit); rounding is to the nearest representable value,
ties to the one with an even last bit.  Written here from that definition,
on float64 values.  Values that would fall below the normal bfloat16 range
or overflow it are outside what the tests produce and are not handled.
"""

import numpy as np


def round_to_bf16(x):
    """float64 array of ``x`` rounded to bfloat16 (nearest, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    sel = np.isfinite(x) & (x != 0.0)
    mant, expo = np.frexp(x[sel])          # x = mant * 2**expo, 0.5 <= |mant| < 1
    kept = np.round(np.ldexp(mant, 8))     # 8 significant bits; numpy rounds half to even
    out[sel] = np.ldexp(kept, expo - 8)
    return out


def store(x, dtype):
    """``x`` as a tensor of ``dtype`` ("fp32" or "bf16") would hold it.  fp32
    storage is taken as exact: the oracle compares fp32 results at
    tolerances far above fp32 rounding."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64)
    raise ValueError("unknown storage dtype %r" % (dtype,))
