"""Pins for the oracle's number formats: OCP E4M3FN (FP8) and bf16.

The FP8 codec is checked against the OCP OFP8 encoding table (tests/golden/e4m3_ocp.json),
against torch's own float8_e4m3fn conversion (an independent library routine), and
against properties any correct round-to-nearest-even codec has (roundtrip, monotone
decode, ties to the even mantissa, saturation).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_matches_ocp_table():
    g = json.load(open(os.path.join(GOLD, "e4m3_ocp.json")))
    for code, val in g["codes"].items():
        got = O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    for code in g["nan_codes"]:
        assert np.isnan(O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0])


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))


def test_e4m3_monotone_and_roundtrip():
    pos = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: all finite non-negative codes
    vals = O.e4m3_decode(pos)
    assert np.all(np.diff(vals) > 0)
    assert vals[-1] == 448.0
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = O.e4m3_encode(O.e4m3_decode(finite).astype(np.float32))
    assert np.array_equal(back, finite)


def test_e4m3_ties_to_even_and_saturation():
    pos = np.arange(0x7E, dtype=np.uint8)  # pairs (c, c+1) up to 0x7D, 0x7E
    lo = O.e4m3_decode(pos)
    hi = O.e4m3_decode(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)  # midpoints are exact in fp32
    got = O.e4m3_encode(mid)
    want = np.where((pos & 1) == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # just below / above a midpoint goes to the nearer neighbour
    below = np.nextafter(mid, np.float32(-np.inf))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(O.e4m3_encode(below[1:]), pos[1:])
    assert np.array_equal(O.e4m3_encode(above), pos + 1)
    sat = O.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, -500.0, -1e30], np.float32))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    tiny = O.e4m3_encode(np.array([2.0 ** -11, 2.0 ** -10, 2.0 ** -10 * 1.0001, -(2.0 ** -9)], np.float32))
    assert list(tiny) == [0x00, 0x00, 0x01, 0x81]  # 2^-10 is the tie between 0 and 2^-9 -> even (0)


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 1, 20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = O.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.normal(0, 1, 5000) * 10.0 ** rng.uniform(-3, 3, 5000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = O.lib()
    ours = np.array([lib.oracle_double_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(ours, ref)
    back = O.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float64).numpy())
