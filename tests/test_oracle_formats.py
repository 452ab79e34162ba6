"""Pins of the oracle's number formats (bf16 and OCP FP8 E4M3) against library
casts and the published format definition; no GPU."""
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties between two bf16 neighbours, both parities of the kept bit
    base = rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    ties = ties[~np.isnan(ties)]          # NaN payloads are not part of the contract
    special = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1e-40, -1e-40, np.inf, -np.inf],
                       dtype=np.float32)
    for v in (a, ties, special):
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.f32_to_bf16_bits(v), ref)


def test_bf16_nan_stays_nan():
    b = O.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(O.bf16_bits_to_f64(b)).all()


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_special_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_decode_published_values():
    for code, val in _golden_e4m3():
        got = O.e4m3_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val, (hex(code), got, val)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    back = O.e4m3_encode(vals[fin].astype(np.float32))
    # +0 and -0 are both exact; every other finite code must come back unchanged
    assert np.array_equal(back, codes[fin])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.uniform(-448, 448, 100_000),
        rng.standard_normal(100_000) * 0.01,
        rng.standard_normal(50_000) * 1e-3,
    ]).astype(np.float32)
    # midpoints between neighbouring codes: ties must go to the even code
    vals = np.sort(np.unique(O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 460.0, 470.0, 1e4, 3e38, -500.0], np.float32)
    assert list(O.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_rounding_helpers_are_two_step():
    # fp64 value just above a bf16 tie after fp32 rounding: rounding straight to bf16
    # would differ from rounding to fp32 first; the oracle must do the latter.
    x = np.float64(1.0) + 2.0 ** -8 + 2.0 ** -40   # fp32 -> 1 + 2^-8 (a bf16 tie) -> 1.0
    assert O.to_bf16(np.array([x]))[0] == 1.0
    assert O.to_bf16(np.array([x]), exact=True)[0] == x


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_rows_properties(seed):
    rng = np.random.default_rng(seed)
    x = O.bf16_bits_to_f64(O.f32_to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32)))
    x[3] = 0.0
    q, s = O.quantize_rows_e4m3(x)
    assert s.dtype == np.float32 and s[3] == 1.0 and not q[3].any()
    dec = O.e4m3_decode(q)
    for r in range(x.shape[0]):
        if r == 3:
            continue
        j = np.argmax(np.abs(x[r]))
        # the row's amax element maps to +-448 (code 0x7E / 0xFE)
        assert q[r, j] & 0x7F == 0x7E
        # each element is within half a step of the e4m3 grid at its magnitude
        y = (x[r] / np.float64(s[r]))
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        half_ulp = 2.0 ** (e - 3) / 2
        assert np.all(np.abs(dec[r] - y) <= half_ulp * (1 + 1e-6) + 1e-7)


def test_quantize_cols_is_rows_of_transpose():
    rng = np.random.default_rng(5)
    w = O.bf16_bits_to_f64(O.f32_to_bf16_bits((rng.standard_normal((3, 32, 48)) * 0.02).astype(np.float32)))
    q, s = O.quantize_cols_e4m3(w)
    assert q.shape == w.shape and s.shape == (3, 48)
    for e in range(3):
        qt, st = O.quantize_rows_e4m3(w[e].T)
        assert np.array_equal(q[e], qt.T) and np.array_equal(s[e], st)
