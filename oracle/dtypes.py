"""Exact conversions between the storage formats and float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Storage conventions used by the oracle:

* ``"f32"``  -- ``numpy.float32`` arrays.
* ``"f16"``  -- IEEE binary16, held either as ``numpy.float16`` or as its
  16-bit patterns in ``numpy.uint16``.
* ``"bf16"`` -- bfloat16 (the top 16 bits of an IEEE binary32), held as
  ``numpy.uint16`` bit patterns (numpy has no bfloat16 type).

Widening to float64 is exact for all three: a binary16 or bfloat16 value is
a binary32 value, and every binary32 value is a binary64 value.

``round_to`` rounds float64 values to the nearest representable value of a
storage format, ties to even, computed from the definition (scale the
significand to the format's precision, ``numpy.rint`` which rounds half to
even, scale back), with the format's subnormal quantum below its smallest
normal and overflow to infinity past the largest finite value plus half an
ulp.  It is used only to judge outputs stored in a 16-bit format.
"""

from __future__ import annotations

import numpy as np

# (significand bits incl. the implicit one, min normal exponent, max finite)
_FORMATS = {
    "f32": (24, -126, float(np.finfo(np.float32).max)),
    "f16": (11, -14, 65504.0),
    "bf16": (8, -126, float.fromhex("0x1.fe00000000000p+127")),
}


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen storage-format values to float64, exactly."""
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError(f"f32 storage must be float32, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "f16":
        if a.dtype == np.uint16:
            a = a.view(np.float16)
        if a.dtype != np.float16:
            raise TypeError(f"f16 storage must be float16/uint16, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError(f"bf16 storage must be uint16 bits, got {a.dtype}")
        # A bfloat16 pattern is the high half of the binary32 pattern.
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest ``dtype`` value (ties to even).

    Returns float64 values that are exactly representable in ``dtype``.
    NaN stays NaN; infinities stay infinite.
    """
    p, emin, fmax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    ax = np.abs(xf)
    # Exponent e with 2**e <= |x| < 2**(e+1); clamp to the normal range so
    # values below the smallest normal use the fixed subnormal quantum.
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one at exact powers of two; correct it.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, emin)
    quantum_exp = (e - (p - 1)).astype(np.int64)
    r = np.ldexp(np.rint(np.ldexp(xf, -quantum_exp)), quantum_exp)
    # Overflow: anything at or beyond max + half an ulp becomes infinite.
    ulp_max = np.ldexp(1.0, int(np.floor(np.log2(fmax))) - (p - 1))
    over = np.abs(r) > fmax
    over |= np.abs(xf) >= fmax + ulp_max / 2
    r = np.where(over, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of ``dtype`` values around |x| (for output checks)."""
    p, emin, _ = _FORMATS[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(0.5, (e - (p - 1)).astype(np.int64))
