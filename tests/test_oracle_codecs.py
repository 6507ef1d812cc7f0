"""Pins for the oracle's number formats (CPU only).

Each encoder/decoder is checked against something other than itself:
library casts (torch, numpy), the OCP E4M3 spec's printed points, and a brute
force nearest-value search.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 1.5, 3.0e38, -3.0e38, 3.3895e38, 3.4e38, np.inf, -np.inf,
            1e-45, -1e-45, 1.17549435e-38, 1.1754942e-38, 65504.0, 65519.0, 65520.0, 6.1e-5,
            5.96e-8, 2.98e-8, 2.99e-8, 1.0 + 2 ** -8, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9,
            1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 448.0, 464.0, 480.0, 0.0009765625]
    return np.array(vals, dtype=np.float32)


def _random_f32(n=200_000, seed=7):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(n).astype(np.float32) * np.float32(3.0)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    b = bits.view(np.float32)
    b = b[np.isfinite(b)]
    return np.concatenate([a, b])


# --------------------------------------------------------------------- decode

def test_e4m3_table_matches_spec_points():
    g = json.load(open(os.path.join(GOLDEN, "e4m3fn_points.json")))
    t = codecs.e4m3fn_table()
    for p in g["points"]:
        code = int(p["code"], 16)
        assert t[code] == p["value"]
        assert np.signbit(t[code]) == np.signbit(p["value"])
    for c in g["nan_codes"]:
        assert np.isnan(t[int(c, 16)])
    assert np.sum(np.isnan(t)) == 2


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = codecs.e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(t))
    assert np.array_equal(ref[~nan], t[~nan])


def test_bf16_f16_decode_match_libraries():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref_bf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got_bf = codecs.bf16_to_f64(bits)
    nan = np.isnan(ref_bf)
    assert np.array_equal(nan, np.isnan(got_bf))
    assert np.array_equal(ref_bf[~nan], got_bf[~nan])
    ref_h = bits.view(np.float16).astype(np.float64)
    got_h = codecs.f16_to_f64(bits)
    nan = np.isnan(ref_h)
    assert np.array_equal(ref_h[~nan], got_h[~nan])


# --------------------------------------------------------------------- encode

def test_bf16_encode_matches_torch():
    x = np.concatenate([_special_f32(), _random_f32()])
    got = codecs.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FFF) == 0x7FC0)


def test_bf16_encode_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)
    got = codecs.f32_to_bf16(x)
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_f16_encode_matches_numpy_and_torch():
    x = np.concatenate([_special_f32(), _random_f32()])
    got = codecs.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    ref_t = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[~nan], ref_t[~nan])
    assert np.all((got[nan] & 0x7FFF) == 0x7E00)


def _e4m3_bruteforce(y):
    """Nearest finite E4M3FN value by exhaustive search; ties to even code;
    saturate beyond 448; NaN -> 0x7F with the sign."""
    t = codecs.e4m3fn_table()
    finite = [c for c in range(256) if not np.isnan(t[c])]
    out = []
    for v in y:
        if np.isnan(v):
            out.append(0xFF if np.signbit(v) else 0x7F)
            continue
        vv = min(max(v, -448.0), 448.0)
        best, bestd = None, None
        for c in finite:
            if (c & 0x80) != (0x80 if np.signbit(vv) else 0):
                continue
            dd = abs(t[c] - vv)
            if bestd is None or dd < bestd or (dd == bestd and (c & 1) == 0 and (best & 1) == 1):
                best, bestd = c, dd
        out.append(best)
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_bruteforce():
    t = codecs.e4m3fn_table()
    pos = np.sort(t[:0x7F])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(3)
    samples = np.concatenate([
        mids, -mids, pos, -pos, mids * (1 + 1e-9), mids * (1 - 1e-9),
        [448.0, 449.0, 463.9, 464.0, 465.0, 480.0, 1e6, np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0,
         2 ** -10, 2 ** -10 * 1.0000001, 3 * 2 ** -10, 2 ** -12],
        rng.standard_normal(3000) * 50, rng.standard_normal(2000) * 0.01,
    ])
    got = codecs.f64_to_e4m3fn(samples)
    ref = _e4m3_bruteforce(samples)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(samples[i], hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_in_range():
    x = _random_f32(100_000, seed=11)
    x = x[np.abs(x) < 464]     # torch's cast is non-saturating beyond this
    got = codecs.f64_to_e4m3fn(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_saturates():
    got = codecs.f64_to_e4m3fn(np.array([464.0, 1e4, np.inf, -500.0, -np.inf]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_scaled_quantisation_uses_correctly_rounded_f32_division():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100_000).astype(np.float32)
    for scale in [2.0 ** -5, 0.0123456, 1.0 / 448.0 * 3.7]:
        got = codecs.f32_to_e4m3fn_scaled(x, scale)
        # fp32 quotient via fp64 then one rounding: correctly rounded for division
        y = (x.astype(np.float64) / np.float64(np.float32(scale))).astype(np.float32)
        ref = torch.from_numpy(y).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, ref), scale


def test_encode_dispatch_roundtrip_exact_values():
    # values already representable in a format survive encode -> decode unchanged
    t = codecs.e4m3fn_table()
    fin = t[~np.isnan(t)].astype(np.float32)
    assert np.array_equal(codecs.decode(codecs.encode(fin, "fp8_e4m3", 1.0), "fp8_e4m3"),
                          fin.astype(np.float64))
    bf = codecs.bf16_to_f64(np.arange(0, 0x7F80, 97, dtype=np.uint16)).astype(np.float32)
    assert np.array_equal(codecs.decode(codecs.encode(bf, "bf16"), "bf16"), bf.astype(np.float64))
