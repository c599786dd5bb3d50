"""OCP 8-bit float E4M3 ("e4m3fn") codec, from the format definition.

[P5] section 7 and [P4] (FP8 KV) store K/V in 8-bit floats with a scale per
head; the pages do not name the encoding, so the OCP E4M3 format is taken:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
exponent field 0, no infinities, and NaN only for exponent=1111 with
mantissa=111.  The largest finite magnitude is 1.75 * 2**8 = 448.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def _decode_one(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 codes (any shape) -> float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("codes must be uint8")
    return _TABLE[c]


def encode_e4m3fn_rne(x) -> np.ndarray:
    """float64 values -> uint8 codes: nearest finite code, ties to even code.

    Values beyond +-448 saturate to +-448 (the inputs are clamped first, as
    the quantiser does); NaN maps to 0x7F.  Brute force over all finite codes
    of the input's sign: slow, but it follows the definition of
    round-to-nearest-even directly.
    """
    v = np.asarray(x, dtype=np.float64)
    flat = v.reshape(-1)
    # Candidates carry the sign of the input, so a value that rounds to zero
    # keeps its sign (-0 is the code 0x80).
    pos_codes = np.arange(0x00, 0x7F, dtype=np.int64)      # 0x7F is NaN
    out = np.empty(flat.shape, dtype=np.uint8)
    chunk = 1 << 16
    for lo in range(0, flat.size, chunk):
        val = flat[lo:lo + chunk]
        nan = np.isnan(val)
        mag = np.minimum(np.abs(np.where(nan, 0.0, val)), E4M3_MAX)
        dist = np.abs(_TABLE[pos_codes][None, :] - mag[:, None])          # [n, 127]
        best = dist.min(axis=1, keepdims=True)
        tie = dist == best
        # at most two neighbouring codes tie; prefer the even one (mantissa LSB 0)
        even = tie & ((pos_codes[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
        code = pos_codes[pick] | np.where(np.signbit(val), 0x80, 0x00)
        out[lo:lo + chunk] = np.where(nan, 0x7F, code).astype(np.uint8)
    return out.reshape(v.shape)
