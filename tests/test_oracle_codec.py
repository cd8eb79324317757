"""Pins of the oracle's NVFP4 codec against things other than itself (CPU only).

* closed forms from the pages: FP4 maximum 6 and 16-entry groups with E4M3 scales
  ([OSFP4] section 1 and appendix D.1), the absmax-to-6 flush of entries 24x below the block
  maximum ([OSFP4] section 1), the positive E4M3 scale set ([OSFP4] appendix I);
* exhaustive decode tables vs a library (torch's float8_e4m3fn) and vs hand enumeration;
* exact brute-force nearest search with Fractions (tests/_brute.py) on tiny inputs,
  including constructed exact ties.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x) -> Fraction:
    return Fraction(float(x))


def test_e2m1_table_matches_hand_enumeration_and_max6():
    hand = _brute.e2m1_codes_table()
    for c, v in hand:
        assert Fraction(O.e2m1_decode(c)) == v, c
    assert max(O.E2M1_MAG_GRID) == 6.0 == O.E2M1_MAX
    # exactly 8 distinct magnitudes, strictly increasing with the code
    assert np.all(np.diff(O.E2M1_MAG_GRID) > 0)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.E4M3_ALL
    both_nan = np.isnan(lib) & np.isnan(mine)
    assert np.all(both_nan | (lib == mine))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x7E] == 448.0 == O.E4M3_MAX
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert np.all(np.diff(O.E4M3_GRID) > 0) and len(O.E4M3_GRID) == 127
    for c, v in _brute.e4m3_nonneg_table():
        assert Fraction(O.E4M3_GRID[c]) == v


def test_e4m3_rounding_of_exact_fp32_values_matches_torch_cast():
    # unit = 1: the quotient is the fp32 value itself; torch's cast is RNE for |x| < 464
    rng = np.random.default_rng(1)
    vals = [0.0, 2.0 ** -10, np.nextafter(2.0 ** -10, 1), 2.0 ** -9, 448.0, 447.0, 3 * 2.0 ** -11]
    mids = (O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2
    for m in mids:
        vals += [m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))]
    vals += list(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(460.0), 4000)))
    x = np.array(vals, dtype=np.float32)
    x = x[x < 464.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = O.rne_grid_index(x.astype(np.float64), 1.0, O.E4M3_GRID)
    assert np.array_equal(got, ref)


def test_e4m3_block_scale_vs_fraction_brute_force():
    """S = nearest E4M3 to the exact A/(6g), ties to even, saturating -- brute force."""
    rng = np.random.default_rng(2)
    table = _brute.e4m3_nonneg_table()
    cases = []
    for _ in range(300):
        g = np.float32(np.exp(rng.uniform(-8, 2)))
        A = np.float32(np.exp(rng.uniform(-14, 9)) * g)
        cases.append((A, g))
    # constructed exact ties: A = 6 g m with m an E4M3 midpoint, g a power of two
    mids = (O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2
    for k in range(0, 126, 5):
        g = np.float32(2.0 ** -3)
        cases.append((np.float32(6 * g * mids[k]), g))
    cases += [(np.float32(0), np.float32(1)), (np.float32(1e30), np.float32(1e-3)),
              (np.float32(6 * 448 * 0.25), np.float32(0.25))]
    A = np.array([c[0] for c in cases], dtype=np.float32)
    g = np.array([c[1] for c in cases], dtype=np.float32)
    got = O.rne_grid_index(A.astype(np.float64), 6.0 * g.astype(np.float64), O.E4M3_GRID)
    for i, (a, gg) in enumerate(cases):
        want = _brute.nearest_code(_f(a) / (6 * _f(gg)), table)
        assert got[i] == want, (a, gg, got[i], want)


def _brute_quantize_row(y32: np.ndarray, g: np.float32):
    table = _brute.e4m3_nonneg_table()
    codes = []
    scales = []
    for b in range(8):
        blk = y32[16 * b:16 * b + 16]
        A = max(abs(_f(v)) for v in blk)
        S = _brute.nearest_code(A / (6 * _f(g)), table)
        sig = dict(table)[S]
        scales.append(S)
        for v in blk:
            codes.append(0 if sig == 0 else _brute.e2m1_encode_brute(_f(v), sig * _f(g)))
    packed = [codes[2 * k] | (codes[2 * k + 1] << 4) for k in range(64)]
    return np.array(packed, dtype=np.uint8), np.array(scales, dtype=np.uint8)


def test_quantize_rows_vs_fraction_brute_force_random_rows():
    rng = np.random.default_rng(3)
    rows = []
    for i in range(12):
        y = rng.standard_normal(128) * np.exp(rng.uniform(-3, 3, 128))
        y[rng.integers(0, 128, 3)] *= 30
        rows.append(y.astype(np.float32))
    rows.append(np.zeros(128, np.float32))                       # all-zero row
    tiny = np.full(128, 1e-30, np.float32)
    tiny[::2] *= -1
    rows.append(tiny)                                             # underflowing scales
    Y = np.stack(rows)
    for g in (np.float32(0.0137), np.float32(1.0), np.float32(2.0 ** -7)):
        codes, scales = O.quantize_rows(Y, g)
        for i in range(len(rows)):
            c_ref, s_ref = _brute_quantize_row(Y[i], g)
            assert np.array_equal(scales[i], s_ref), (i, g)
            assert np.array_equal(codes[i], c_ref), (i, g)


def test_e2m1_constructed_ties_and_midpoints():
    """Every E2M1 midpoint hit exactly, and one fp32 ulp either side, in a block whose scale
    is exactly representable (A = 6 * sigma * g)."""
    g = np.float32(0.5)
    sigma = 3.0                                     # E4M3 code 0x44
    A = np.float32(6 * sigma * g)
    unit = sigma * float(g)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        x = np.float32(m * unit)
        vals += [x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(100))]
    vals = vals[:15]
    row_vals = [A] + vals                            # first element sets the block max
    y = np.zeros(128, np.float32)
    y[:16] = np.array(row_vals, np.float32)
    y[16:32] = -y[:16]
    codes, scales = O.quantize_rows(y[None], g)
    assert scales[0, 0] == 0x44 and O.E4M3_ALL[0x44] == 3.0
    c_ref, s_ref = _brute_quantize_row(y, g)
    assert np.array_equal(codes[0], c_ref) and np.array_equal(scales[0], s_ref)
    nib = O.unpack_nibbles(codes[0])
    # ties go to the even code: 0.25->0, 0.75->1.0(code2), 1.25->1.0, 1.75->2.0(code4),
    # 2.5->2.0, 3.5->4.0(code6), 5->4.0
    tie_codes = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for i, m in enumerate(mids[:5]):
        assert nib[1 + 3 * i] == tie_codes[m], m
        assert nib[16 + 1 + 3 * i] == (0 if tie_codes[m] == 0 else tie_codes[m] | 8), m


def test_flush_below_one_24th_of_block_max():
    """absmax-to-6: with a representable block scale, |y| < A/24 -> 0, |y| = A/24 -> 0 (tie to
    even), just above A/24 -> +-0.5 ([OSFP4] section 1: entries 24x smaller are zeroed)."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    ratio = facts["absmax_to_6_flush_ratio"]["value"]
    assert ratio == 24 == 4 * O.E2M1_MAX       # 6 / 0.25: the first midpoint
    for g, sigma in [(np.float32(1.0), 1.0), (np.float32(0.03125), 7.0), (np.float32(2.0 ** -5), 448.0)]:
        A = np.float32(6 * sigma * float(g))
        thr = np.float32(A / ratio)
        assert float(thr) * ratio == float(A)
        y = np.zeros(128, np.float32)
        y[0] = A
        y[1] = thr
        y[2] = np.nextafter(thr, np.float32(0))
        y[3] = np.nextafter(thr, np.float32(1e9))
        y[4] = -np.nextafter(thr, np.float32(1e9))
        y[5] = -thr
        codes, scales = O.quantize_rows(y[None], g)
        nib = O.unpack_nibbles(codes[0])
        assert O.E4M3_ALL[scales[0, 0]] == sigma
        assert nib[0] == 7                            # block max maps to 6
        assert nib[1] == 0 and nib[2] == 0 and nib[5] == 0
        assert nib[3] == 1 and nib[4] == 9            # +0.5 and -0.5


def test_saturation():
    g = np.float32(1e-3)
    y = np.zeros(128, np.float32)
    y[:16] = 1e6                                     # A/(6g) far above 448 -> 0x7E
    codes, scales = O.quantize_rows(y[None], g)
    assert scales[0, 0] == 0x7E
    assert np.all(O.unpack_nibbles(codes[0])[:16] == 7)
    # values above 6*sigma*g inside a block whose scale rounded down -> code 7
    g = np.float32(1.0)
    y = np.zeros(128, np.float32)
    y[0] = np.float32(6 * 8.25)                      # A/(6g) = 8.25 rounds down to the E4M3 value 8
    codes, scales = O.quantize_rows(y[None], g)
    assert O.E4M3_ALL[scales[0, 0]] == 8.0
    assert O.unpack_nibbles(codes[0])[0] == 7


def test_zero_block_and_signed_zero():
    y = np.zeros(128, np.float32)
    y[17] = -0.0
    y[20] = 1.0
    codes, scales = O.quantize_rows(y[None], np.float32(1.0))
    assert scales[0, 0] == 0 and np.all(O.unpack_nibbles(codes[0])[:16] == 0)
    assert O.unpack_nibbles(codes[0])[17] == 0                   # -0 stored as +0 code


def test_dequantize_exact_and_roundtrip_error_bound():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((50, 128)) * 3).astype(np.float32)
    g = np.float32(np.abs(y).max() / 2688)
    codes, scales = O.quantize_rows(y, g)
    xh = O.dequantize(codes, scales, g)
    # exactness: every dequantised value equals the Fraction product
    nib = O.unpack_nibbles(codes)
    for i in range(3):
        for j in range(0, 128, 7):
            v = dict(_brute.e2m1_codes_table())[int(nib[i, j])]
            s = dict(_brute.e4m3_nonneg_table())[int(scales[i, j // 16])]
            assert Fraction(xh[i, j]) == v * s * _f(g)
    # E2M1 half-step bound: |x - xhat| <= (spacing/2) * sigma * g, spacing <= 2 at the top
    sig = O.E4M3_ALL[scales.astype(np.int64)].repeat(16, axis=1)
    assert np.all(np.abs(xh - y) <= 1.0 * sig * float(g) + 1e-30)
