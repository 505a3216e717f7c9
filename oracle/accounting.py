"""Storage accounting (oracle).

Sources:
  * Together AI OSCAR page, summary and "Results": 2.28 bits per KV element;
    "Serving system": BF16 sink (64) and recent (256) windows are 0.24% of the
    tokens at 128K.
  * Qiita article, "Fix 1": an INT2 element is 0.25 byte; "Why 256K was
    abandoned": the INT2 KV costs 8.0 KiB per token for 16 full-attention
    layers x 4 KV heads and 2.5 KiB for 10 layers x 2 KV heads (head_dim 256).

Pins (tests/test_oracle_accounting.py): the page's 8.0 / 2.5 KiB and 0.24%
figures as golden values; the 3.00-bit history cost of G = 32 with fp16
scale and zero.
"""

from __future__ import annotations


def int2_code_bytes_per_token(layers: int, kv_heads: int, head_dim: int) -> float:
    """Bytes of packed INT2 codes for K and V of one token (no scales)."""
    return layers * kv_heads * head_dim * 2 * 0.25


def bf16_share(L: int, sink: int = 64, recent: int = 256) -> float:
    """Fraction of the L cached tokens that sit in the BF16 windows."""
    return min(L, sink + recent) / L


def bits_per_element(L: int, head_dim: int = 128, group_size: int = 32,
                     meta_bits_per_group: int = 32, sink: int = 64,
                     recent: int = 256) -> float:
    """Average stored bits per K/V element for a cache of length L."""
    bf16 = min(L, sink + recent)
    hist = L - bf16
    per_hist = 2.0 + meta_bits_per_group / group_size
    return (hist * per_hist + bf16 * 16.0) / L
