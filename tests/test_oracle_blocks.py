"""Pins for oracle.blocks (GGUF Q8_0 / Q4_0 decoding) -- CPU only.

The decode is exact in f32 (an fp16 scale has 11 significant bits, |q| <= 128
has 8), so every expected value below is a closed form on hand-built bytes.
"""
import struct

import numpy as np
import pytest

from oracle import blocks


def q8_block(d_bits, qs):
    return struct.pack("<H", d_bits) + bytes(np.asarray(qs, dtype=np.int8).tobytes())


def q4_block(d_bits, payload):
    return struct.pack("<H", d_bits) + bytes(payload)


def test_f16_decode_matches_ieee_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    mine = blocks._f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(mine[~np.isnan(mine)]), np.signbit(ref[~np.isnan(ref)]))


def test_q8_0_half_scale_every_int():
    qs = np.arange(-127, 128)  # 255 values -> 8 blocks (last one padded below)
    qs = np.concatenate([qs, np.zeros(1, int)]).reshape(8, 32)
    raw = b"".join(q8_block(0x3800, r) for r in qs)  # 0x3800 = 0.5
    w = blocks.dequant_q8_0(np.frombuffer(raw, np.uint8), 1, 256)
    assert w.dtype == np.float32
    assert np.array_equal(w.reshape(-1), (0.5 * qs.reshape(-1)).astype(np.float32))


def test_q8_0_subnormal_and_negative_scales():
    qs = np.arange(-16, 16)
    raw = q8_block(0x0001, qs) + q8_block(0xB800, qs) + q8_block(0x7BFF, qs)
    w = blocks.dequant_q8_0(np.frombuffer(raw, np.uint8), 3, 32)
    assert np.array_equal(w[0], (qs * 2.0 ** -24).astype(np.float32))    # smallest subnormal
    assert np.array_equal(w[1], (qs * -0.5).astype(np.float32))          # negative scale
    assert np.array_equal(w[2], (qs * 65504.0).astype(np.float32))       # largest finite fp16


def test_q8_0_int8_extremes():
    qs = np.array([-128, 127] * 16)
    w = blocks.dequant_q8_0(np.frombuffer(q8_block(0x3C00, qs), np.uint8), 1, 32)  # d = 1
    assert np.array_equal(w[0], qs.astype(np.float32))


def test_q4_0_nibble_order():
    # byte j: low nibble j, high nibble 15 - j -> element j = j - 8, element j+16 = 7 - j
    payload = [(j & 15) | ((15 - j) << 4) for j in range(16)]
    w = blocks.dequant_q4_0(np.frombuffer(q4_block(0x4000, payload), np.uint8), 1, 32)  # d = 2
    want = np.array([2.0 * (j - 8) for j in range(16)] + [2.0 * (7 - j) for j in range(16)], np.float32)
    assert np.array_equal(w[0], want)


def test_q4_0_offset_eight_and_subnormal_scale():
    payload = [0x88] * 16  # every nibble 8 -> value 0
    w = blocks.dequant_q4_0(np.frombuffer(q4_block(0x3C00, payload), np.uint8), 1, 32)
    assert np.array_equal(w[0], np.zeros(32, np.float32))
    payload = [0x0F] * 16  # low nibble 15 -> +7, high nibble 0 -> -8
    w = blocks.dequant_q4_0(np.frombuffer(q4_block(0x0001, payload), np.uint8), 1, 32)
    assert np.array_equal(w[0], np.array([7.0] * 16 + [-8.0] * 16, np.float32) * np.float32(2.0 ** -24))


def test_padded_row_keeps_logical_columns():
    # 40 logical columns -> 2 blocks per row; the padded tail is dropped
    rows = []
    for r in range(3):
        rows.append(q8_block(0x3C00, np.arange(32) - 16 + r) + q8_block(0x3800, np.full(32, r + 1)))
    w = blocks.dequant_q8_0(np.frombuffer(b"".join(rows), np.uint8), 3, 40)
    assert w.shape == (3, 40)
    for r in range(3):
        assert np.array_equal(w[r, :32], (np.arange(32) - 16 + r).astype(np.float32))
        assert np.array_equal(w[r, 32:], np.full(8, 0.5 * (r + 1), np.float32))


def test_wrong_byte_count_is_refused():
    with pytest.raises(ValueError):
        blocks.dequant_q8_0(np.zeros(33, np.uint8), 1, 32)
    with pytest.raises(ValueError):
        blocks.dequant_q4_0(np.zeros(34, np.uint8), 1, 32)
    with pytest.raises(ValueError):
        blocks.dequant(3, np.zeros(4, np.uint8), 1, 1)


def test_scales_finite_detects_inf_and_nan():
    ok = q8_block(0x3C00, np.zeros(32))
    inf = q8_block(0x7C00, np.zeros(32))
    nan = q4_block(0x7E00, [0] * 16)
    assert blocks.scales_finite(8, np.frombuffer(ok, np.uint8), 1, 32)
    assert not blocks.scales_finite(8, np.frombuffer(ok + inf, np.uint8), 2, 32)
    assert not blocks.scales_finite(2, np.frombuffer(nan, np.uint8), 1, 32)


def test_f32_tensor_passthrough():
    x = np.arange(12, dtype=np.float32).reshape(3, 4) - 5.5
    assert np.array_equal(blocks.dequant(0, x.view(np.uint8).reshape(-1), 3, 4), x)


# ---------------------------------------------------------------- K-quants
def q4_k_golden():
    """One Q4_K super-block laid out by hand: d = 1 (fp16 0x3C00), dmin = 0.5
    (0x3800); (scale, min) of sub-blocks 0..7 = (1,0) (2,1) (3,2) (4,3) (5,32)
    (6,33) (7,62) (63,63), packed into the 12 scale bytes
    01 02 03 C4 80 81 C2 C3 05 16 E7 FF; quant byte 32c + l holds l % 16 in its
    low nibble (sub-block 2c) and 15 - l % 16 in its high one (2c + 1)."""
    sb = bytearray(144)
    sb[0:4] = bytes([0x00, 0x3C, 0x00, 0x38])
    sb[4:16] = bytes([0x01, 0x02, 0x03, 0xC4, 0x80, 0x81, 0xC2, 0xC3, 0x05, 0x16, 0xE7, 0xFF])
    for c in range(4):
        for l in range(32):
            sb[16 + 32 * c + l] = (l % 16) | ((15 - l % 16) << 4)
    return np.frombuffer(bytes(sb), np.uint8)


def test_q4_k_hand_laid_super_block():
    w = blocks.dequant(blocks.T_Q4_K, q4_k_golden(), 1, 256)[0]
    # value = 1 * scale * q - 0.5 * min, worked out by hand per position
    want = {0: 0.0, 5: 5.0, 32: 2 * 15 - 0.5, 67: 3 * 3 - 1.0, 113: 4 * 14 - 1.5, 128: -16.0,
            162: 6 * 13 - 16.5, 223: 7 * 15 - 31.0, 224: 63 * 15 - 31.5, 255: -31.5}
    for i, v in want.items():
        assert w[i] == v, i


def q6_k_golden():
    """One Q6_K super-block laid out by hand: d = 0.5, scales = -8..7, and
    value i holds q = i % 64 (so q - 32 runs -32..31 in each quarter): the low
    bytes carry l & 15 in both nibbles, the high byte of l carries l >> 4,
    2 + (l >> 4), l >> 4, 2 + (l >> 4) in its four 2-bit fields."""
    sb = bytearray(210)
    for h in range(2):
        for l in range(32):
            sb[64 * h + l] = (l & 15) | ((l & 15) << 4)
            sb[64 * h + 32 + l] = (l & 15) | ((l & 15) << 4)
            sb[128 + 32 * h + l] = (l >> 4) | ((2 + (l >> 4)) << 2) | ((l >> 4) << 4) | ((2 + (l >> 4)) << 6)
    sb[192:208] = bytes([(i - 8) & 0xFF for i in range(16)])
    sb[208:210] = bytes([0x00, 0x38])
    return np.frombuffer(bytes(sb), np.uint8)


def test_q6_k_hand_laid_super_block():
    w = blocks.dequant(blocks.T_Q6_K, q6_k_golden(), 1, 256)[0]
    # value = 0.5 * scale[i // 16] * (i % 64 - 32), worked out by hand
    want = {0: 128.0, 17: 52.5, 40: -24.0, 63: -77.5, 64: 64.0, 127: -15.5, 128: 0.0, 200: -48.0, 255: 108.5}
    for i, v in want.items():
        assert w[i] == v, i


@pytest.mark.parametrize("ttype,rms", [(blocks.T_Q4_K, 0.1), (blocks.T_Q6_K, 0.025)])
def test_k_quant_round_trip_of_the_input_encoder(ttype, rms):
    """The synthetic-input encoder (written separately from the layout's
    packing rules) and the decoder agree: decoded values are within the
    quantisation step of the encoded ones (a swapped nibble, scale or half
    would give errors of the signal's own size)."""
    import synth
    x = (0.02 * np.random.default_rng(3).standard_normal((8, 1024))).astype(np.float32)
    w = blocks.dequant(ttype, synth.encode(ttype, x), 8, 1024)
    assert np.sqrt(np.mean((w - x) ** 2)) < rms * np.std(x)


def test_k_quant_scales_finite_and_row_length():
    g = q4_k_golden().copy()
    assert blocks.scales_finite(blocks.T_Q4_K, g, 1, 256)
    g[3] = 0x7C  # dmin = inf
    assert not blocks.scales_finite(blocks.T_Q4_K, g, 1, 256)
    h = q6_k_golden().copy()
    h[209] = 0x7E  # d = nan
    assert not blocks.scales_finite(blocks.T_Q6_K, h, 1, 256)
    with pytest.raises(ValueError, match="256"):
        blocks.dequant(blocks.T_Q4_K, np.zeros(144, np.uint8), 1, 128)
