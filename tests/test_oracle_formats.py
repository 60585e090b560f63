"""Pins for the oracle's byte decoders (e4m3fn, ue8m0, bf16).

Each decoder is checked over every code against torch's own casts (a library
implementation independent of the oracle's bit arithmetic) and against closed-form
values of the formats (DeepSeek-V4.1-Flash-NVFP4 model.py module globals name e4m3 data
with ue8m0 scales).
"""
import math

import numpy as np
import torch


def test_e4m3_all_codes_match_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = orc.decode_e4m3(np.arange(256))
    for c in range(256):
        if math.isnan(lib[c]):
            assert math.isnan(ours[c]), c
        else:
            assert ours[c] == lib[c], (hex(c), ours[c], lib[c])


def test_e4m3_closed_forms(orc):
    v = orc.e4m3_value
    assert v(0x7E) == 448.0              # largest finite
    assert v(0xFE) == -448.0
    assert v(0x38) == 1.0                # exponent field 7 = bias
    assert v(0xB8) == -1.0
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    # one mantissa step at exponent 0 is 1/8
    assert v(0x39) == 1.125


def test_e8m0_all_codes(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(255):
        assert orc.e8m0_value(c) == 2.0 ** (c - 127) == lib[c], c
    assert math.isnan(orc.e8m0_value(255)) and math.isnan(lib[255])


def test_bf16_all_codes_match_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([orc.bf16_value(int(b)) for b in bits])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


# OCP Microscaling Formats (MX) v1.0, element type FP4 (E2M1): magnitudes of codes 0-7
# written out from the format's definition (2 exponent bits, bias 1, 1 mantissa bit,
# exponent 0 subnormal); code + 8 is the negative.  No library here decodes fp4, so the
# table is the independent side.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes_match_table(orc):
    for c in range(16):
        want = E2M1_TABLE[c & 7] * (-1.0 if c & 8 else 1.0)
        got = orc.e2m1_value(c)
        assert got == want, (c, got, want)
        assert math.copysign(1.0, got) == (-1.0 if c & 8 else 1.0), c
    # only the low four bits are a code: the byte's other nibble is the neighbour element
    assert orc.e2m1_value(0x07) == 6.0 and orc.e2m1_value(0x0F) == -6.0


def test_e2m1_values_are_exact_e4m3_values():
    # every fp4 value survives torch's e4m3 cast unchanged, which is what lets the
    # indexer pins compare the two formats on shared values
    vals = torch.tensor(E2M1_TABLE + [-v for v in E2M1_TABLE], dtype=torch.float64)
    back = vals.to(torch.float8_e4m3fn).to(torch.float64)
    assert torch.equal(back, vals)
