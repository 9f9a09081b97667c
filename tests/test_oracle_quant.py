"""Pins of the oracle's bf16 helpers, packing and quantizer (CPU only).

Each pin checks the oracle against something other than itself: worked words and worked
groups written by hand (tests/golden/), a library conversion (torch's bf16 cast), brute
force over every bf16 pattern, exact rational arithmetic, and the error bound the
quantizer must meet.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, quant
from workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = bf16.to_f64(b)
    ok = np.isfinite(v)
    return b[ok], v[ok]


# ---------------------------------------------------------------- bf16 helpers

def test_bf16_widening_is_exact():
    b = np.array([0x3F80, 0xBF80, 0x4300, 0x0001, 0x7F7F, 0x3EA0], np.uint16)
    assert list(bf16.to_f64(b)) == [1.0, -1.0, 128.0, 2.0 ** -133, 3.3895313892515355e38, 0.3125]


def test_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
                        # exact ties: bf16 value + half an ulp
                        ((rng.integers(0x3000, 0x4F00, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.rne(x), ref)


def test_roundup_is_smallest_bf16_not_below():
    bits, vals = _all_finite_bf16()
    order = np.argsort(vals, kind="stable")
    sv, sb = vals[order], bits[order]
    rng = np.random.default_rng(2)
    x = np.concatenate([np.abs(rng.standard_normal(50000)).astype(np.float32),
                        rng.uniform(0, 1e-3, 50000).astype(np.float32),
                        bf16.to_f32(rng.integers(0, 0x7F00, 1000).astype(np.uint16))])
    got = bf16.to_f64(bf16.roundup(x))
    idx = np.searchsorted(sv, x.astype(np.float64), side="left")
    assert np.array_equal(got, sv[idx])
    # representable inputs are returned unchanged
    exact = bf16.to_f32(np.array([0x3F80, 0x3C01, 0x0001], np.uint16))
    assert np.array_equal(bf16.roundup(exact), np.array([0x3F80, 0x3C01, 0x0001], np.uint16))


# ---------------------------------------------------------------- packing

def test_packing_worked_words():
    cases = json.load(open(os.path.join(GOLDEN, "packing.json")))["cases"]
    for c in cases:
        codes = np.array(c["codes"], np.uint32)[None]
        word = int(c["word"], 16)
        assert int(quant.pack(codes, c["bits"])[0, 0]) == word, c
        assert list(quant.unpack(np.array([[word]], np.uint32), c["bits"])[0]) == c["codes"], c


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_straddling_widths_pack_as_one_bit_stream(bits):
    """Widths that do not divide 32: the row's codes as one little-endian bit stream, built
    here as a Python integer (sum of code_i << (bits * i)) and cut into 32-bit words; a code
    whose bits cross a word boundary keeps its low bits in the lower word."""
    rng = np.random.default_rng(100 + bits)
    for D in (32, 64, 256):
        codes = rng.integers(0, 1 << bits, size=D)
        stream = 0
        for i, c in enumerate(codes):
            stream |= int(c) << (bits * i)
        want = [(stream >> (32 * k)) & 0xFFFFFFFF for k in range(D * bits // 32)]
        got = quant.pack(codes.astype(np.uint32)[None], bits)[0]
        assert [int(x) for x in got] == want
        assert np.array_equal(quant.unpack(got[None], bits)[0], codes.astype(np.uint32))
    # a hand-worked 3-bit row: codes 0..7, 0, 1, 2, ... -> word 0 holds codes 0..9 in bits 0..29
    # and the low two bits of code 10 (= 2, binary 10) in bits 30..31
    if bits == 3:
        codes = (np.arange(32) % 8).astype(np.uint32)[None]
        w0 = sum(c << (3 * i) for i, c in enumerate([0, 1, 2, 3, 4, 5, 6, 7, 0, 1])) | (2 << 30)
        assert int(quant.pack(codes, 3)[0, 0]) == w0 == 0x88FAC688
        assert int(quant.pack(codes, 3)[0, 1]) == (2 >> 2) | (3 << 1) | (4 << 4) | (5 << 7) | (6 << 10) | (
            7 << 13) | (0 << 16) | (1 << 19) | (2 << 22) | (3 << 25) | (4 << 28) | ((5 & 1) << 31)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_unpack_round_trip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(7, 3, 256)).astype(np.uint32)
    words = quant.pack(codes, bits)
    assert words.shape == (7, 3, 256 * bits // 32)
    assert np.array_equal(quant.unpack(words, bits), codes)
    # and the other way round: any word survives unpack -> pack (rows of whole codes)
    w = rng.integers(0, 1 << 32, size=(5, 8 * bits), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(quant.pack(quant.unpack(w, bits), bits), w)


# ---------------------------------------------------------------- quantizer

def _group_from_pattern(pattern, bits):
    d = np.arange(64)
    if pattern == "d % 16":
        x = (d % 16).astype(np.float32)
    elif pattern == "d / 4":
        x = (d / 4).astype(np.float32)
    elif pattern == "alternate -1, 1":
        x = np.where(d % 2 == 0, -1.0, 1.0).astype(np.float32)
    elif pattern == "d % 4":
        x = (d % 4).astype(np.float32)
    elif pattern == "constant 0.3125":
        x = np.full(64, 0.3125, np.float32)
    else:
        raise ValueError(pattern)
    return x


def test_quantizer_worked_groups():
    cases = json.load(open(os.path.join(GOLDEN, "quant_examples.json")))["cases"]
    for c in cases:
        bits = c["bits"]
        if "pattern" in c:
            x = _group_from_pattern(c["pattern"], bits)
        else:
            x = np.full(64, c["fill"], np.float32)
            x[: len(c["values_head"])] = c["values_head"]
        xb = bf16.rne(x)
        assert np.array_equal(bf16.to_f32(xb), x)          # every value is exactly bf16
        codes, s, b = quant.quantize_codes(xb[None], bits)
        assert int(s[0, 0]) == int(c["scale_bits"], 16), c["name"]
        assert int(b[0, 0]) == int(c["bias_bits"], 16), c["name"]
        codes = codes[0]
        if c.get("codes") == "d % 16":
            assert np.array_equal(codes, np.arange(64) % 16)
        elif c.get("codes") == "d % 4":
            assert np.array_equal(codes, np.arange(64) % 4)
        elif c.get("codes") == "0":
            assert not codes.any()
            deq = quant.dequantize(quant.pack(codes[None], bits), s, b, bits)
            assert np.array_equal(deq[0], x.astype(np.float64))
        if "codes_head" in c:
            assert list(codes[: len(c["codes_head"])]) == c["codes_head"], c["name"]
        for k, v in c.get("codes_at", {}).items():
            assert int(codes[int(k)]) == v, (c["name"], k)


def _half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_quantizer_against_exact_rationals(bits):
    """Brute force in exact arithmetic: scale is the smallest bf16 >= RN32((max-min)/n), and each
    code is round-half-even of the exact quotient, except where the exact quotient lies within
    f32 rounding of a tie (there the f32 division the reading prescribes decides)."""
    rng = np.random.default_rng(10 + bits)
    xb = bf16.rne(rng.standard_normal((40, 64)).astype(np.float32) * rng.uniform(0.1, 10, (40, 1)).astype(np.float32))
    codes, s, b = quant.quantize_codes(xb, bits)
    n = (1 << bits) - 1
    bits_all, vals_all = _all_finite_bf16()
    for r in range(xb.shape[0]):
        x = [Fraction(float(v)) for v in bf16.to_f64(xb[r])]
        mx, mn = max(x), min(x)
        s32 = np.float32(np.float32(float(mx - mn)) / np.float32(n))   # the reading's f32 steps
        cand = vals_all[vals_all >= float(s32)]
        assert float(bf16.to_f64(s[r, 0])) == cand.min()
        assert Fraction(float(bf16.to_f64(b[r, 0]))) == mn
        sc = Fraction(float(bf16.to_f64(s[r, 0])))
        for d in range(64):
            qx = (x[d] - mn) / sc
            want = min(max(_half_even(qx), 0), n)
            frac = qx - (qx.numerator // qx.denominator)
            near_tie = abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20) * max(1, qx)
            if not near_tie:
                assert int(codes[r, d]) == want, (r, d, float(qx))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("wl", ["c3", "c5", "c2"])
@pytest.mark.parametrize("group", [64, 32, 128])
def test_quantize_error_bound(bits, wl, group):
    """|x - dequant(quant(x))| <= scale / 2 for every element; codes within [0, 2^bits - 1];
    the group minimum maps to code 0 and the maximum to the top code (bits <= 4) or within
    2 of it (5, 6 and 8 bits, where the rounded-up scale can leave the top code unused)."""
    w = make_workload(wl, B=2, len_lo=300, len_hi=400, D=256, HK=2)
    k, v = w.kv(0)
    for x in (k, v):
        words, s, bb = quant.quantize(x, bits, group)
        codes = quant.unpack(words, bits)
        n = (1 << bits) - 1
        assert codes.max() <= n
        xf = bf16.to_f64(x)
        deq = quant.dequantize(words, s, bb, bits, group)
        half = np.repeat(bf16.to_f64(s), group, axis=-1) / 2
        assert np.all(np.abs(xf - deq) <= half)
        g = xf.reshape(xf.shape[:-1] + (256 // group, group))
        cg = codes.reshape(g.shape)
        amin, amax = g.argmin(-1), g.argmax(-1)
        assert np.all(np.take_along_axis(cg, amin[..., None], -1) == 0)
        top = np.take_along_axis(cg, amax[..., None], -1)
        if bits <= 4:
            assert np.all(top == n)
        else:
            assert np.all(top >= n - 2)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_group_size_is_a_partition_of_the_row(bits):
    """Scale groups are independent: quantizing a row with groups of G equals quantizing each
    G-element slice as a one-group row (checked for G = 32, 64, 128 against G = slice length), and
    the packed words do not depend on the grouping beyond the codes themselves."""
    rng = np.random.default_rng(40 + bits)
    x = bf16.rne(rng.standard_normal((6, 256)).astype(np.float32) * 3)
    for G in (32, 64, 128):
        codes, s, b = quant.quantize_codes(x, bits, G)
        for gi in range(256 // G):
            c1, s1, b1 = quant.quantize_codes(x[:, gi * G:(gi + 1) * G], bits, G)
            assert np.array_equal(codes[:, gi * G:(gi + 1) * G], c1)
            assert np.array_equal(s[:, gi], s1[:, 0]) and np.array_equal(b[:, gi], b1[:, 0])
        words, _, _ = quant.quantize(x, bits, G)
        assert np.array_equal(words, quant.pack(codes, bits))


def test_effective_bytes_ratio_from_the_page_header():
    """kvq4-decode.ts (inference 1.0.0 diff page 50, file header): 4-bit group-64 K/V with
    scales costs ~0.28x of bf16 bytes per token at head dim 256; exactly 144/512 per row."""
    assert quant.bytes_per_token_head(4, 256) / quant.bytes_per_token_head(16, 256) == 0.28125
    assert quant.bytes_per_token_head(4, 256) == 288
    assert quant.bytes_per_token_head(16, 128) == 512
    assert quant.bytes_per_token_head(8, 128) == 272
    assert quant.bytes_per_token_head(2, 128) == 80
