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


def test_bits_of_every_record_layout_match_the_record_sizes():
    """Bits per history element from the head-record sizes of the pool format
    (64 code bytes + (s, z) bytes per 128-channel K and V pair): 96 B -> 3.0,
    80 B -> 2.5, 72 B -> 2.25 (G = 128 fp16, and G = 64 with 8-bit s and z);
    the two 72-byte layouts give the OSCAR page's 2.28 at 128K."""
    from oracle import cache
    for G, sb, hist_bits in ((32, 16, 3.0), (64, 16, 2.5), (128, 16, 2.25), (64, 8, 2.25)):
        lay = cache.Layout(128, G, 1, 1, 64, 256, 1, 1, sb)
        assert lay.head_record_bytes * 8 / (2 * 128) == hist_bits
        meta = 2 * sb                                       # s and z per group
        assert accounting.bits_per_element(10 ** 12, group_size=G, meta_bits_per_group=meta) == \
            hist_bits + 320 * (16 - hist_bits) / 10 ** 12
    b = accounting.bits_per_element(131072, group_size=64, meta_bits_per_group=16)
    assert round(b, 2) == 2.28
