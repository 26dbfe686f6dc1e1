"""Pins of the fp8 row-quantiser definition (CPU only): the E4M3 format
(OCP FP8, largest finite 448) decoded from its definition, round to nearest
even on worked ties, the minimality of the power-of-two row scale, and the
half-ulp error bound."""

import numpy as np
import torch

from oracle import quant


def test_e4m3_decode_definition():
    # 1.0 = exponent 7 (bias 7), 448 = 1.75 * 2^8, smallest subnormal 2^-9, NaN at 0x7F
    assert quant.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x00, 0xB8, 0x40, 0x30]))[:7].tolist() == [
        1.0, 448.0, 2.0 ** -9, 0.0, -1.0, 2.0, 0.5]
    assert np.isnan(quant.e4m3_decode(np.array([0x7F]))[0])
    # every finite code round-trips through the library cast
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = quant.e4m3_decode(codes).astype(np.float32)
    back = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = ~((codes == 0x80))  # -0 encodes as 0x80 and decodes to -0.0 == 0.0
    assert np.array_equal(back[ok], codes[ok])


def test_round_to_nearest_even_ties():
    # the row maximum 76 sets the scale 2^-2 (76 * 4 = 304 <= 448 < 608), so the
    # scaled row is 4.25, 4.75, 272, 304: ties at spacing 0.5 in [4, 8) and 32 in
    # [256, 512); to even: 4.25 -> 4 (000), 4.75 -> 5 (010), 272 -> 256 (000), 304 -> 320 (010)
    codes, sc = quant.quantize_rows(np.array([[1.0625, 1.1875, 68.0, 76.0, 1.0, 0.0, 0.0, 0.0]], np.float32))
    assert sc[0] == 127 - 2
    assert quant.e4m3_decode(codes[0, :4]).tolist() == [4.0, 5.0, 256.0, 320.0]
    assert quant.dequantize_rows(codes, sc)[0, :4].tolist() == [1.0, 1.25, 64.0, 80.0]


def test_scale_is_the_smallest_power_of_two():
    g = np.random.default_rng(3)
    x = (g.standard_normal((200, 64)) * 10.0 ** g.uniform(-6, 6, (200, 1))).astype(np.float32)
    codes, sc = quant.quantize_rows(x)
    for r in range(200):
        e = int(sc[r]) - 127
        amax = float(np.abs(x[r]).max())
        assert amax * 2.0 ** -e <= 448.0 < amax * 2.0 ** -(e - 1)
    assert quant.row_exponent(448.0) == 0 and quant.row_exponent(449.0) == 1
    assert quant.row_exponent(224.0) == -1 and quant.row_exponent(1.0) == -8
    assert quant.row_exponent(2.0 ** -130) == -127  # clamped to the smallest E8M0 scale
    zc, zs = quant.quantize_rows(np.zeros((1, 64), np.float32))
    assert zs[0] == 127 and not zc.any()


def test_half_ulp_error_bound():
    g = np.random.default_rng(4)
    x = (g.standard_normal((100, 128)) * 10.0 ** g.uniform(-3, 3, (100, 1))).astype(np.float32)
    codes, sc = quant.quantize_rows(x)
    deq = quant.dequantize_rows(codes, sc)
    scale = np.ldexp(1.0, sc.astype(np.int64) - 127)[:, None]
    y = np.abs(x) / scale
    normal = y >= 2.0 ** -6
    # normal range: |error| <= half a unit in the last place = 2^-4 relative
    assert (np.abs(deq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-12)).all()
    # subnormal range: absolute spacing 2^-9 of the scaled value
    assert (np.abs(deq - x)[~normal] <= 2.0 ** -10 * scale.repeat(128, 1)[~normal] * (1 + 1e-12)).all()
