"""KV cache size in bytes.

[P1] section 3.1, [P4] (byte formula), [P5] section 1, [P3] section 3.2 and
[P2] section 1.1 all give the same count: for every token, every layer keeps
one K and one V vector per KV head, so

    bytes per token = 2 * layers * kv_heads * head_dim * bytes_per_element

and a whole cache is that times the tokens per sequence times the batch.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

from fractions import Fraction


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_element) -> Fraction:
    # Fraction keeps sub-byte formats (int4 ~ 0.5 byte) exact.
    return 2 * layers * kv_heads * head_dim * Fraction(bytes_per_element)


def kv_bytes(layers: int, kv_heads: int, head_dim: int, bytes_per_element,
             tokens: int, batch: int = 1) -> Fraction:
    return kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_element) * tokens * batch
