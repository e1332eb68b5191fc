"""Pins for the oracle's bf16 and OCP E4M3 converters and its 1x128 activation quantiser.

They are checked against torch's own converters (an independent implementation) and against values
fixed by the IEEE-754 / OCP 8-bit floating point definitions.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def test_bf16_round_matches_torch(oracle):
    g = torch.Generator().manual_seed(1)
    v = torch.cat([torch.randn(20000, generator=g) * 10 ** torch.randint(-30, 30, (20000,), generator=g).float(),
                   torch.tensor([0.0, -0.0, 1.0, -1.0, 1e-40, -3e-39, 3.3e38, 1.00390625, 1.01171875])])
    ref = v.to(torch.bfloat16).float()
    got = torch.tensor([oracle.round_bf16(float(a)) for a in v.tolist()])
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


def test_bf16_round_ties_from_double(oracle):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.  Just above the tie rounds up.
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6          # tie, odd below -> up
    assert oracle.round_bf16(2.0 ** -133) == 2.0 ** -133                        # smallest subnormal
    assert oracle.round_bf16(2.0 ** -134) == 0.0                                # tie to even (0)
    assert oracle.round_bf16(-(2.0 ** -134) * 1.5) == -(2.0 ** -133)


# OCP E4M3: a few values fixed by the definition (bias 7, 3 mantissa bits, max 448, 0x7F NaN).
OCP_E4M3_POINTS = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
                   0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x80: -0.0, 0xFE: -448.0}


def test_e4m3_decode_definition_points(oracle):
    for c, v in OCP_E4M3_POINTS.items():
        assert oracle.e4m3_decode(c) == v, hex(c)
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))


def test_e4m3_decode_all_codes_match_torch(oracle):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().double()
    for c in range(256):
        a, b = oracle.e4m3_decode(c), float(ref[c])
        assert (math.isnan(a) and math.isnan(b)) or a == b, hex(c)


def test_e4m3_encode_matches_torch_in_range(oracle):
    # every finite bf16 value with |v| <= 448, plus random fp32 values
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    bits = bits[torch.isfinite(bits) & (bits.abs() <= 448)]
    g = torch.Generator().manual_seed(2)
    rnd = (torch.rand(100000, generator=g) * 2 - 1) * 448 * torch.rand(100000, generator=g) ** 6
    v = torch.cat([bits, rnd])
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8)
    got = torch.tensor([oracle.e4m3_encode(float(a)) for a in v.tolist()], dtype=torch.uint8)
    mism = (ref != got).nonzero().flatten()
    assert mism.numel() == 0, [(float(v[i]), int(ref[i]), int(got[i])) for i in mism[:5]]


def test_e4m3_encode_saturates(oracle):
    # OCP saturating conversion: every magnitude above 448 maps to +-448, never NaN.
    for v in [448.0001, 463.9, 464.0, 500.0, 1e6, 1e30]:
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE


def test_e4m3_encode_ties_to_even(oracle):
    assert oracle.e4m3_encode(1.0625) == 0x38      # halfway 1 .. 1.125 -> even mantissa (1.0)
    assert oracle.e4m3_encode(1.1875) == 0x3A      # halfway 1.125 .. 1.25 -> 1.25
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # halfway 0 .. 2^-9 -> 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02


def test_quantize_rows_rule(oracle):
    g = torch.Generator().manual_seed(3)
    v = torch.randn(7, 384, generator=g) * torch.logspace(-3, 3, 7)[:, None]
    v[3, 128:256] = 0.0                                     # an all-zero group
    q, s = oracle.quantize_rows_e4m3(v.numpy())
    dec = torch.tensor(q).view(torch.float8_e4m3fn).float()
    for r in range(7):
        for gi in range(3):
            grp = v[r, gi * 128:(gi + 1) * 128]
            amax = grp.abs().max()
            if amax == 0:
                assert s[r, gi] == 1.0 and (q[r, gi * 128:(gi + 1) * 128] == 0).all()
                continue
            assert s[r, gi] == np.float32(amax.item()) / np.float32(448.0)
            assert dec[r, gi * 128:(gi + 1) * 128].abs().max() == 448.0     # the group max maps to 448
            # per-element error of the dequantised value: half an E4M3 ulp (relative 2^-4), or the
            # subnormal quantum below 2^-6
            deq = dec[r, gi * 128:(gi + 1) * 128].double() * float(s[r, gi])
            err = (deq - grp.double()).abs()
            bound = torch.maximum(grp.double().abs() * 2.0 ** -4, torch.tensor(2.0 ** -10 * float(s[r, gi])))
            assert (err <= bound * (1 + 1e-6)).all()
