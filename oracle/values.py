"""Exact float64 values of stored cache / query elements.

Every storage format used here embeds exactly in float64, so the oracle works
on the very values the device reads:
  * f32 and f16: numpy's own widening;
  * bf16: the 16 stored bits are the top half of an fp32 word;
  * fp8 e4m3fn: the OCP definition in fp8_e4m3.py;
  * int8: the two's-complement integer (a symmetric quantised code).

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from .fp8_e4m3 import decode_e4m3fn

STORAGE_NUMPY = {
    "f32": np.float32,
    "f16": np.float16,
    "bf16": np.uint16,        # raw bits
    "fp8_e4m3": np.uint8,     # raw codes
    "int8": np.int8,          # symmetric integer codes
}


def stored_to_f64(a, tag: str) -> np.ndarray:
    a = np.asarray(a)
    want = STORAGE_NUMPY[tag]
    if a.dtype != want:
        raise TypeError(f"{tag} values must be passed as {np.dtype(want).name}, got {a.dtype}")
    if tag in ("f32", "f16", "int8"):
        return a.astype(np.float64)
    if tag == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return decode_e4m3fn(a)
