"""Pins of the oracle's number formats and FP8 latent-row quantizer.

The oracle decodes/encodes E4M3 and bf16 from their definitions; here it is
checked against values fixed by the format definition, against torch's own
float8_e4m3fn / bfloat16 conversions (an independent library), and against a
brute-force nearest-grid-point search written with exact fractions.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    """All finite E4M3 values, built by enumerating (exponent, mantissa)."""
    vals = {}
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            vals[(e << 3) | m] = mag
    return vals


def test_decode_definition_values(orc):
    with open(os.path.join(GOLDEN, "e4m3_definition_values.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for code_hex, val in rows:
        got = float(orc.e4m3_decode(np.array([int(code_hex, 16)], np.uint8))[0])
        if val == "nan":
            assert math.isnan(got), code_hex
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code_hex, got)


def test_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert nan.sum() == 2                                   # 0x7F and 0xFF
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_torch(orc):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(4096, generator=g) * torch.exp2(torch.randint(-30, 30, (4096,), generator=g).float()))
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.bf16_decode(bits), b.to(torch.float64).numpy())


def _nearest_even(x: float):
    """Brute force: nearest finite E4M3 magnitude, ties to even mantissa, saturate."""
    grid = _grid()
    xa = abs(Fraction(x))
    best = None
    for code, mag in grid.items():
        d = abs(mag - xa)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code)
    code = best[1]
    if xa >= 448:
        code = 0x7E
    if math.copysign(1.0, x) < 0:
        code |= 0x80
    return code


def test_encode_bruteforce_nearest(orc):
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(300).astype(np.float32) * np.float32(50))
    xs += list((rng.standard_normal(200) * 2.0 ** -8).astype(np.float32))      # subnormal range
    grid = sorted(set(float(v) for v in _grid().values()))
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]                    # exact ties
    xs += [np.float32(m) for m in mids] + [np.float32(-m) for m in mids[::7]]
    xs += [np.float32(v) for v in (0.0, -0.0, 448.0, 449.0, 464.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11)]
    xs = np.array(xs, dtype=np.float32)
    got = orc.e4m3_encode(xs)
    for x, c in zip(xs, got):
        assert c == _nearest_even(float(x)), (float(x), hex(c), hex(_nearest_even(float(x))))


def test_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_encode(x), ref)


def test_kv_quantize_closed_forms(orc):
    rng = np.random.default_rng(3)
    rows = torch.from_numpy(rng.standard_normal((64, 576)).astype(np.float32)).to(torch.bfloat16)
    rows[5] = 0.0
    bits = rows.view(torch.int16).numpy().view(np.uint16)
    codes, scales = orc.kv_quantize(bits)
    x = rows.to(torch.float64).numpy()
    # all-zero row: scale 1, all codes +0
    assert scales[5] == 1.0 and (codes[5] == 0).all()
    for r in range(64):
        if r == 5:
            continue
        amax = np.abs(x[r]).max()
        assert scales[r] == np.float32(np.float32(amax) / np.float32(448.0))
        # the largest-magnitude element lands on +-448
        j = int(np.abs(x[r]).argmax())
        assert codes[r, j] & 0x7F == 0x7E
        # dequantized row is within half a grid step of the input
        deq = orc.e4m3_decode(codes[r]) * float(scales[r])
        y = np.abs(x[r]) / float(scales[r])
        step_y = np.maximum(np.exp2(np.floor(np.log2(np.maximum(y, 1e-30))) - 3), 2.0 ** -9)
        assert (np.abs(deq - x[r]) <= step_y * float(scales[r]) * 0.5 * (1 + 1e-5)).all()


def test_kv_quantize_matches_torch_division_and_cast(orc):
    rng = np.random.default_rng(4)
    rows = torch.from_numpy(rng.standard_normal((128, 576)).astype(np.float32)).to(torch.bfloat16)
    codes, scales = orc.kv_quantize(rows.view(torch.int16).numpy().view(np.uint16))
    xf = rows.to(torch.float32)
    sc = xf.abs().amax(dim=1) / 448.0
    ref = (xf / sc[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(scales, sc.numpy())
    np.testing.assert_array_equal(codes, ref)
