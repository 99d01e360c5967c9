"""Pins for the oracle's scalar decoders and row dequantizers.

Each test ties the oracle to something other than itself: values printed on
the pages (tests/golden/*.json, each entry cited), closed forms evaluated in
exact rational arithmetic (tests/exact.py), exhaustive enumeration against
torch's float8 dtypes and numpy's float16, and brute force on tiny inputs.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact import round_f32, same_f32, frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ E2M1

def test_e2m1_codebook_exhaustive():
    g = golden("e2m1_codebook.json")
    for code, want in enumerate(g["values"]):
        got = oracle.e2m1(code)
        assert got == want
        assert math.copysign(1.0, got) == math.copysign(1.0, want), code


def test_e2m1_page_facts():
    g = golden("e2m1_codebook.json")
    for f in g["facts"]:
        got = oracle.e2m1(f["code"])
        assert got == f["e2m1"]
        if f.get("negative_zero"):
            assert got == 0.0 and math.copysign(1.0, got) < 0
        if "unsigned" in f:
            assert f["code"] == f["unsigned"]


def test_e2m1_is_not_twos_complement():
    # Four Bits, Three Contracts, section 1: reading the nibble as signed INT4
    # gives a different number. The two readings agree only on code 0 (zero)
    # and, by coincidence, code 13 (-3).
    agree = {c for c in range(16) if oracle.e2m1(c) == oracle.int4_sym_value(c)}
    assert agree == {0, 13}


# ------------------------------------------------------------------ E8M0

def test_e8m0_facts_and_closed_form():
    g = golden("scales.json")["e8m0"]
    assert oracle.e8m0(g[0]["byte"]) == g[0]["value"]
    assert math.isnan(oracle.e8m0(g[1]["byte"]))
    for b in range(255):
        assert oracle.e8m0(b) == math.ldexp(1.0, b - 127)


def test_e8m0_exhaustive_vs_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e8m0(b)
        if math.isnan(t[b]):
            assert math.isnan(got), b
        else:
            assert got == t[b], b


# ------------------------------------------------------------------ E4M3FN

def test_e4m3fn_facts():
    for f in golden("scales.json")["e4m3fn"]:
        if "byte" in f:
            assert oracle.e4m3fn(f["byte"]) == f["value"], f
        if "nan_bytes" in f:
            nans = [b for b in range(256) if math.isnan(oracle.e4m3fn(b))]
            assert nans == f["nan_bytes"]


def test_e4m3fn_exhaustive_vs_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3fn(b)
        if math.isnan(t[b]):
            assert math.isnan(got), b
        else:
            assert got == t[b], b
            assert math.copysign(1.0, got) == math.copysign(1.0, t[b]), b
    finite = [abs(oracle.e4m3fn(b)) for b in range(256) if not math.isnan(oracle.e4m3fn(b))]
    assert max(finite) == 448.0
    assert sum(1 for b in range(256) if not math.isnan(oracle.e4m3fn(b))) == 254


# ------------------------------------------------------------------ fp16 / bf16

def test_f16_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536):
        got = oracle.f16(b)
        r = ref[b]
        if math.isnan(r):
            assert math.isnan(got), b
        else:
            assert got == r and math.copysign(1.0, got) == math.copysign(1.0, r), b


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 1e-45, 1.0 + 2**-8, 1.0 + 3 * 2**-8,
                  1.0 + 2**-8 + 2**-20], dtype=np.float32),
        rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(vals)
    got_vec = oracle.bf16_rne_array(vals)
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(got_vec, got)
    # NaN stays NaN
    assert all(math.isnan(oracle.bf16_value(int(b))) for b in got[nan])


# ------------------------------------------------------------------ MXFP4 rows

def _pack_low_even(codes):
    codes = list(codes)
    assert len(codes) % 2 == 0
    return np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)], dtype=np.uint8)


def test_mxfp4_dot_fact_in_a_block():
    g = golden("fp4_examples.json")["mxfp4_dot"]
    for case in g["cases"]:
        codes = [oracle.e2m1_nearest(w, case["scale"]) for w in g["w"]]
        codes32 = codes + [0] * 28
        row = oracle.dequant_rows(oracle.MXFP4, _pack_low_even(codes32)[None, :],
                                  np.array([[case["e8m0"]]], np.uint8), 1.0, 32, [0])[0]
        assert row[:4].tolist() == case["recon"]
        x = np.zeros(32, np.float32)
        x[:4] = g["x"]
        y, s = oracle.gemv_rows(oracle.MXFP4, _pack_low_even(codes32)[None, :],
                                np.array([[case["e8m0"]]], np.uint8), 1.0, 32, x, [0])
        assert y[0] == case["dot"]
    assert abs(sum(a * b for a, b in zip(g["w"], g["x"])) - g["exact_dot"]) < 1e-12


def test_scale_grids_and_nearest():
    g = golden("fp4_examples.json")["scale_grids"]
    assert sorted({oracle.e2m1(c) * 0.5 for c in range(8)}) == g["grid_0_5"]
    assert max(oracle.e2m1(c) * 0.125 for c in range(16)) == g["max_0_125"]
    for f in g["nearest"]:
        assert oracle.e2m1(oracle.e2m1_nearest(f["w"], f["scale"])) * f["scale"] == f["recon"]


def test_mxfp4_closed_form_every_code_and_scale_byte():
    # Every (code, scale byte) pair: w = E2M1(code) * 2^(b-127), exact or +-inf.
    codes = np.arange(16, dtype=np.uint8)
    cb = golden("e2m1_codebook.json")["values"]
    for b in range(255):
        row = oracle.dequant_rows(oracle.MXFP4, _pack_low_even(list(codes) * 2)[None, :],
                                  np.array([[b]], np.uint8), 1.0, 32, [0])[0]
        for i in range(32):
            want = round_f32(Fraction(cb[i % 16]) * Fraction(2) ** (b - 127),
                             negative_zero=(i % 16 == 8))
            assert same_f32(row[i], want), (b, i)


def test_mxfp4_group_and_row_indexing():
    # distinct scale per (row, group): a wrong group or row stride changes values
    n, k = 3, 96
    codes = np.full((n, k // 2), 0x22, np.uint8)  # every element code 2 -> 1.0
    scales = np.array([[120 + 3 * r + gi for gi in range(3)] for r in range(n)], np.uint8)
    out = oracle.dequant_rows(oracle.MXFP4, codes, scales, 1.0, k, [2, 0, 1])
    for oi, r in enumerate([2, 0, 1]):
        for i in range(k):
            assert out[oi, i] == math.ldexp(1.0, int(scales[r, i // 32]) - 127)


# ------------------------------------------------------------------ NVFP4 rows

def test_nvfp4_muser_fixture_bit_exact():
    g = golden("nvfp4_fixture.json")
    row = oracle.dequant_rows(oracle.NVFP4, np.array([g["packed"]], np.uint8),
                              np.array([[g["scale_byte"]]], np.uint8), g["scale2"], 16, [0])[0]
    for got, want in zip(row.tolist(), g["values"]):
        assert same_f32(got, want)


def test_nvfp4_page_examples():
    g = golden("fp4_examples.json")
    ex = [e for e in g["block_scale_examples"]]
    inv = {oracle.e2m1(c): c for c in range(16) if c != 8}
    for e in ex:
        vals = e.get("values", [e.get("value")])
        codes = [inv[v] for v in vals]
        codes += [0] * (16 - len(codes)) if e["fmt"] == "nvfp4" else [0] * (32 - len(codes))
        expect = e["expect"] if isinstance(e["expect"], list) else [e["expect"]]
        if e["fmt"] == "nvfp4":
            row = oracle.dequant_rows(oracle.NVFP4, _pack_low_even(codes)[None, :],
                                      np.array([[e["scale_byte"]]], np.uint8), e["scale2"], 16, [0])[0]
        else:
            row = oracle.dequant_rows(oracle.MXFP4, _pack_low_even(codes)[None, :],
                                      np.array([[e["scale_byte"]]], np.uint8), 1.0, 32, [0])[0]
        assert row[:len(expect)].tolist() == expect, e["cite"]
    s = golden("scales.json")["e4m3fn"][-1]["nvfp4"]
    row = oracle.dequant_rows(oracle.NVFP4, _pack_low_even([s["code"]] + [0] * 15)[None, :],
                              np.array([[s["scale_byte"]]], np.uint8), s["scale2"], 16, [0])[0]
    assert row[0] == s["value"]


def test_nvfp4_exhaustive_every_finite_scale_byte_and_code():
    # All 254 finite E4M3FN bytes x 16 codes, against the exact product rounded
    # once to binary32; scale2 chosen so that the final rounding is inexact.
    cb = golden("e2m1_codebook.json")["values"]
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = [b for b in range(256) if b not in (0x7F, 0xFF)]
    codes = _pack_low_even(list(range(16)))
    for scale2 in (np.float32(0.01), np.float32(0.25), np.float32(3.0e-39)):
        data = np.tile(codes, (len(finite), 1))
        scales = np.array(finite, np.uint8)[:, None]
        out = oracle.dequant_rows(oracle.NVFP4, data, scales, float(scale2), 16, list(range(len(finite))))
        for ri, b in enumerate(finite):
            for c in range(16):
                exact = Fraction(cb[c]) * Fraction(float(t[b])) * frac(scale2)
                # a zero product carries the exclusive-or of the factors' signs
                neg = (math.copysign(1, cb[c]) < 0) != (math.copysign(1, t[b]) < 0)
                want = round_f32(exact, negative_zero=neg)
                assert same_f32(out[ri, c], want), (b, c, float(scale2))


def test_nvfp4_pinned_order_differs_from_regrouped():
    # (e2m1*e4m3fn)*scale2 rounds once; e2m1*(e4m3fn*scale2) may round twice.
    # Find a case where the two orders disagree and check the oracle follows the
    # pinned one (Chapter 7, sections 7.1 and 7.2).
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    found = 0
    rng = np.random.default_rng(3)
    for scale2 in rng.uniform(0.001, 1.0, 400).astype(np.float32):
        for b in (0x29, 0x3B, 0x46, 0x2F):
            c = 13  # -3.0
            pinned = np.float32(np.float32(-3.0 * t[b]) * scale2)
            regrouped = np.float32(np.float32(-3.0) * np.float32(np.float32(t[b]) * scale2))
            if pinned != regrouped:
                row = oracle.dequant_rows(oracle.NVFP4, _pack_low_even([c] + [0] * 15)[None, :],
                                          np.array([[b]], np.uint8), float(scale2), 16, [0])[0]
                assert row[0] == pinned and row[0] != regrouped
                found += 1
    assert found > 0


def test_nvfp4_group_of_16_indexing():
    n, k = 2, 64
    codes = np.full((n, k // 2), 0x44, np.uint8)  # code 4 -> 2.0
    scales = np.array([[0x38 + 8 * gi + r for gi in range(4)] for r in range(n)], np.uint8)
    out = oracle.dequant_rows(oracle.NVFP4, codes, scales, 1.0, k, [1, 0])
    for oi, r in enumerate([1, 0]):
        for i in range(k):
            assert out[oi, i] == 2.0 * oracle.e4m3fn(int(scales[r, i // 16]))
