"""Pins of oracle.accounting (closed forms and the pages' figures)."""

from oracle import accounting


def test_history_bits_group32_fp16_meta():
    # 2 code bits + (16-bit s + 16-bit z) / 32 channels = 3 bits
    assert accounting.bits_per_element(10 ** 9) == 3.0 + (320 * 13.0) / 10 ** 9


def test_bits_reading_of_2_28():
    """0.25 bit of metadata per element (e.g. G = 128 with fp16 s and z) plus the
    BF16 windows gives ~2.28 bits at 128K, the OSCAR page's figure."""
    b = accounting.bits_per_element(131072, group_size=128, meta_bits_per_group=32)
    assert round(b, 2) == 2.28


def test_all_bf16_when_short():
    assert accounting.bits_per_element(320) == 16.0
    assert accounting.bf16_share(100) == 1.0
