"""Exact decoding of stored values, and rounding to the storage type.

The layer stores state in the workload's type only in the KV pages (the
appended K/V of this step).  Rounding there is round-to-nearest-even.
"""
import numpy as np

_BF16_SHIFT = 45                      # 52 - 7 fraction bits dropped from binary64
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_STEP = 2.0 ** -133
_BF16_OVERFLOW = 2.0 ** 128


def to_f64(a, dtype: str) -> np.ndarray:
    """Exact value of a stored array: bf16 bit patterns (uint16) or float32."""
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_f64(v, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest value of the storage type (ties to even); result in fp64."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = np.ascontiguousarray(v).view(np.uint64)
    lsb = (u >> np.uint64(_BF16_SHIFT)) & np.uint64(1)
    bias = np.uint64((1 << (_BF16_SHIFT - 1)) - 1) + lsb
    r = ((u + bias) & ~np.uint64((1 << _BF16_SHIFT) - 1)).view(np.float64).copy()
    tiny = np.abs(v) < _BF16_MIN_NORMAL
    if tiny.any():
        r[tiny] = np.round(v[tiny] / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP
    big = np.abs(r) >= _BF16_OVERFLOW
    if big.any():
        r[big] = np.copysign(np.inf, v[big])
    nan = np.isnan(v)
    if nan.any():
        r[nan] = np.nan
    return r


def encode(v, dtype: str) -> np.ndarray:
    """fp64 values that are exactly representable in the storage type -> stored array."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    if dtype == "f32":
        return f
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
