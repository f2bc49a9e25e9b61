"""Pins of the oracle's format codecs against the format definitions and against
independent implementations (torch's bf16 / float8_e4m3fn casts, the e2m1 value
list printed on the chenxutan.com page, section 6.2)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    got = O.decode_rows(codes, O.BF16, 65536).reshape(-1)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_bf16_encode_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
    ])
    # exact halfway points between neighbouring bf16 values (ties to even)
    base = rng.integers(0, 0x7F7F, 3000).astype(np.uint32) << 16  # finite bf16 values
    half = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, half, -half])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got, _ = O.encode_rows(x.astype(np.float64), O.BF16, x.size)
    assert np.array_equal(got.view(np.uint16).reshape(-1), ref)


def test_e4m3_decode_all_codes_match_torch_and_definition():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.decode_rows(codes, O.KV_PACKED, 256, 0).reshape(-1)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.array_equal(ref[~nan], got[~nan])
    assert O.e4m3_decode(0x7E) == 448.0          # largest finite
    assert O.e4m3_decode(0x01) == 2.0 ** -9      # smallest subnormal
    assert O.e4m3_decode(0x08) == 2.0 ** -6      # smallest normal


def test_e4m3_encode_rne_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0)])
    # midpoints between adjacent finite codes (ties to even), both signs
    vals = np.array([O.e4m3_decode(c) for c in range(0x7E + 1)])
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    assert O.e4m3_encode(500.0) == 0x7E
    assert O.e4m3_encode(1e9) == 0x7E
    assert O.e4m3_encode(-1e9) == 0xFE
    assert O.e4m3_encode(464.0) == 0x7E  # halfway to the next (non-existent) step


def _gold_e2m1():
    vals = {}
    with open(os.path.join(GOLD, "e2m1_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def test_e2m1_decode_matches_page_value_list():
    gold = _gold_e2m1()
    assert len(gold) == 8
    for c in range(16):
        want = gold[c & 7] * (-1.0 if c & 8 else 1.0)
        assert O.e2m1_decode(c) == want
        if want != 0.0:
            assert O.e2m1_encode(want) == c


@pytest.mark.parametrize("x,val", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                                   (3.5, 4.0), (5.0, 4.0), (5.5, 6.0), (7.0, 6.0), (100.0, 6.0),
                                   (-0.75, -1.0), (-5.0, -4.0), (0.2, 0.0), (0.3, 0.5)])
def test_e2m1_encode_rne_and_saturation(x, val):
    assert O.e2m1_decode(O.e2m1_encode(x)) == val


def test_e8m0_decode():
    assert O.e8m0_decode(127) == 1.0
    assert O.e8m0_decode(0) == 2.0 ** -127
    assert O.e8m0_decode(254) == 2.0 ** 127
    assert math.isnan(O.e8m0_decode(255))


def test_mx_block_exponent_is_smallest_covering_power():
    rng = np.random.default_rng(3)
    amaxes = np.concatenate([np.exp(rng.uniform(-20, 20, 4000)),
                             [6.0, 3.0, 1.5, 0.75, 6.0 * 2 ** 5, 6.0 * 2 ** -7]])
    for a in amaxes:
        e = O.mx_block_exponent(a)
        assert 6.0 * 2.0 ** e >= a
        assert 6.0 * 2.0 ** (e - 1) < a
    assert O.mx_block_exponent(6.0) == 0
    assert O.mx_block_exponent(6.0 * (1 + 2 ** -30)) == 1
    assert O.mx_block_exponent(3.0) == -1
    assert O.mx_block_exponent(0.0) == -127


def test_mxfp4_row_roundtrip_and_nibble_order():
    gold = _gold_e2m1()
    grid = np.array([gold[i] for i in range(8)])
    rng = np.random.default_rng(4)
    for e in (-3, 0, 2, 7):
        v = rng.choice(np.concatenate([grid, -grid]), size=(5, 64)) * 2.0 ** e
        v[:, 0] = 6.0 * 2.0 ** e  # every block reaches the top of its range
        v[:, 32] = -6.0 * 2.0 ** e
        codes, scales = O.encode_rows(v, O.MXFP4, 64)
        assert np.all(scales == 127 + e)
        back = O.decode_rows(codes, O.MXFP4, 64, scales=scales)
        assert np.array_equal(back, v)
    # element 0 in the low nibble, element 1 in the high nibble
    row = np.zeros((1, 32))
    row[0, 0], row[0, 1] = 0.5, 6.0
    codes, scales = O.encode_rows(row, O.MXFP4, 32)
    assert scales[0, 0] == 127 and codes[0, 0] == 0x71


def test_mxfp4_quantization_error_bound():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((200, 128))
    codes, scales = O.encode_rows(v, O.MXFP4, 128)
    back = O.decode_rows(codes, O.MXFP4, 128, scales=scales)
    blk_scale = 2.0 ** (scales.astype(np.float64) - 127)
    step = np.repeat(blk_scale, 32, axis=1)
    # e2m1 spacing is at most 2 (between 4 and 6) -> error <= 1 * scale
    assert np.all(np.abs(back - v) <= step * 1.0 + 1e-15)


def test_packed_row_layout():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((7, 512))
    packed, _ = O.encode_rows(v, O.KV_PACKED, 512, 64)
    assert packed.shape == (7, 576)
    lo = torch.from_numpy(v[:, :64].astype(np.float32)).to(torch.bfloat16).view(torch.uint8).numpy()
    hi = torch.from_numpy(v[:, 64:].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # encode from fp32-representable inputs equals torch's casts byte for byte
    v32 = v.astype(np.float32).astype(np.float64)
    packed32, _ = O.encode_rows(v32, O.KV_PACKED, 512, 64)
    assert np.array_equal(packed32[:, :128], lo.reshape(7, 128))
    assert np.array_equal(packed32[:, 128:], hi.reshape(7, 448))
