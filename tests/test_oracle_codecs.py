"""Pins for the oracle's number formats (CPU only).

Each format is pinned to something other than the oracle itself: hand-worked
fixtures under tests/golden (from the bit layouts), torch's library casts
(float8_e4m3fn, bfloat16) and closed-form properties.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line.split()


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)]) \
        and np.array_equal(np.signbit(a[~np.isnan(a)]), np.signbit(b[~np.isnan(b)]))


def test_e4m3_golden_points():
    for code, val in _rows("e4m3_points.txt"):
        got = oracle.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert _same([got], [float(val)]), (code, got, val)


def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(oracle.e4m3_decode_table(), ref)


def test_e4m3_encode_golden_ties():
    for val, code in _rows("e4m3_rounding.txt"):
        got = oracle.e4m3_encode_rne(np.array([float(val)]))[0]
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.uniform(-0.05, 0.05, 200_000),          # subnormal / small-normal band
        rng.standard_normal(200_000) * 30,
    ]).astype(np.float32)
    # every exact midpoint between neighbouring finite codes (the RNE ties)
    tab = oracle.e4m3_decode_table()
    pos = np.sort(tab[(tab >= 0) & ~np.isnan(tab)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, -mids, pos.astype(np.float32)])
    vals = np.clip(vals, -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_rne(vals)
    assert np.array_equal(got, ref)


def test_e4m3_roundtrip_all_finite_codes():
    tab = oracle.e4m3_decode_table()
    finite = np.nonzero(~np.isnan(tab))[0].astype(np.uint8)
    assert np.array_equal(oracle.e4m3_encode_rne(tab[finite]), finite)


def test_e4m3_saturates():
    assert oracle.e4m3_encode_rne(np.array([1e6, -1e6, 449.0]))[0] == 0x7E
    assert oracle.e4m3_encode_rne(np.array([-1e6]))[0] == 0xFE


def test_e2m1_golden_table():
    tab = oracle.e2m1_decode_table()
    for nib, val in _rows("e2m1_points.txt"):
        assert _same([tab[int(nib)]], [float(val)])


def test_e2m1_unpack_order_low_nibble_first():
    packed = np.array([[0x21, 0x7F]], dtype=np.uint8)    # elements 1, 2 (=0.5, 1.0) then 15, 7
    got = oracle.e2m1_unpack_decode(packed)
    assert got.tolist() == [[0.5, 1.0, -6.0, 6.0]]


def test_ue8m0_golden_points():
    for code, val in _rows("ue8m0_points.txt"):
        got = oracle.ue8m0_decode(np.array([int(code)]))[0]
        assert _same([got], [float(val)]), (code, got, val)


def test_ue8m0_code_is_smallest_nonsaturating_power_of_two():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.abs(rng.standard_normal(50_000)) * 10.0 ** rng.uniform(-6, 6, 50_000),
                           448.0 * 2.0 ** np.arange(-20, 20)]).astype(np.float32)
    code = oracle.ue8m0_code_for_amax(amax, 448.0).astype(np.int64)
    scale = np.ldexp(1.0, code - 127)
    ratio = amax.astype(np.float64) / scale
    # amax/scale lands in (224, 448]: the scale is the smallest power of two not saturating 448
    assert np.all(ratio <= 448.0 * (1 + 2 ** -23))
    assert np.all(ratio > 224.0 * (1 - 2 ** -23))
    # exact powers of two times 448 map exactly
    exact = 448.0 * 2.0 ** np.arange(-20, 20)
    c2 = oracle.ue8m0_code_for_amax(exact.astype(np.float32), 448.0).astype(np.int64)
    assert np.array_equal(c2, 127 + np.arange(-20, 20))
    assert oracle.ue8m0_code_for_amax(np.array([0.0], dtype=np.float32), 448.0)[0] == 0


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(300_000) * 10.0 ** rng.uniform(-30, 30, 300_000),
                           np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38])]).astype(np.float32)
    # ties: values exactly halfway between two bf16 numbers
    base = rng.integers(0, 2 ** 15, 20_000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    vals = np.concatenate([vals, ties])
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits_rne(vals)
    assert np.array_equal(got, ref)
    back = oracle.bf16_bits_to_f32(got)
    assert np.array_equal(back, torch.from_numpy(vals).to(torch.bfloat16).float().numpy())
