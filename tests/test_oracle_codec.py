"""Pins for the oracle's K8/V4 codec (CPU only).

Every check here compares the oracle with something other than itself:
hand-derived golden cases, closed forms, an independent exact-rational
implementation of each rounding step, and the reconstruction bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec
from tests import exact_fp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_cases.json")


def _pad(row, n):
    out = np.zeros(n, np.float32)
    out[: len(row)] = np.asarray(row, np.float32)
    return out


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden_cases(case):
    if case["kind"] == "k":
        x = _pad(case["x"], 64)
        c, s = codec.quantize_k(x[None])
        assert list(c[0, : len(case["x"])]) == case["codes"]
        assert np.all(c[0, len(case["x"]):] == 0)
        assert int(s[0]) == int(case["scale_bits"], 16)
    else:
        if "x_groups" in case:
            groups, codes = case["x_groups"], case["codes_groups"]
        else:
            groups, codes = [case["x"]], [case["codes"]]
        D = 32 * max(2, len(groups))
        x = np.zeros(D, np.float32)
        for g, row in enumerate(groups):
            x[32 * g: 32 * g + len(row)] = row
        c, s = codec.quantize_v(x[None])
        for g, exp in enumerate(codes):
            assert list(c[0, 32 * g: 32 * g + len(exp)]) == exp
        for g, bits in enumerate(case["scale_bits"]):
            assert int(s[0, g]) == int(bits, 16)


def test_lossless_closed_form():
    """x = c * s with fp16 s and one |c| at the maximum: codes and scale come
    back exactly."""
    rng = np.random.default_rng(11)
    for qmax, fn, D in ((127, codec.quantize_k, 128), (7, codec.quantize_v, 32)):
        for _ in range(200):
            e = int(rng.integers(-14, 10))
            mant = int(rng.integers(1024, 2048))
            s = np.float32(np.float16(mant * 2.0 ** (e - 10)))
            c = rng.integers(-qmax, qmax + 1, size=D)
            c[int(rng.integers(0, D))] = qmax * (1 if rng.random() < 0.5 else -1)
            x = (c.astype(np.float32) * s).astype(np.float32)
            codes, sb = fn(x[None])
            assert np.array_equal(codes[0], c.astype(np.int8))
            assert np.all(np.asarray(sb).ravel()[0] == np.float16(s).view(np.uint16))


def _rand_rows(rng, n, d):
    rows = []
    for _ in range(n):
        mag = 10.0 ** rng.uniform(-9, 7)
        r = (rng.standard_normal(d) * mag).astype(np.float32)
        if rng.random() < 0.2:       # make ties likely: multiples of a half-scale
            a = np.float32(np.max(np.abs(r)))
            r[: d // 2] = (np.round(r[: d // 2] / a * 254) / 254 * a).astype(np.float32)
        rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_matches_exact_rational_rounding(kind):
    """Scale and codes equal an exact-rational evaluation of the same rule
    (fp32 division, RNE to fp16 with saturation, fp32 division, RNE to int)."""
    rng = np.random.default_rng(5 if kind == "k" else 6)
    d, qmax = (64, 127) if kind == "k" else (32, 7)
    x = _rand_rows(rng, 60, d)
    if kind == "k":
        codes, sb = codec.quantize_k(x)
    else:
        codes, sb = codec.quantize_v(x)
        sb = sb[:, 0]
    for i in range(x.shape[0]):
        a = float(np.max(np.abs(x[i])))
        s = exact_fp.codec_scale(a, qmax)
        assert Fraction(float(np.uint16(sb[i]).view(np.float16))) == s
        for j in range(d):
            assert int(codes[i, j]) == exact_fp.codec_code(float(x[i, j]), s, qmax)


def test_scale_brute_force_over_all_fp16():
    """For a 2-element row the chosen scale is the fp16 nearest (ties even)
    to fp32(a/127): brute force over every finite positive fp16 value."""
    all16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    rng = np.random.default_rng(7)
    for _ in range(300):
        a = np.float32(10.0 ** rng.uniform(-8, 6.5))
        _, sb = codec.quantize_k(np.array([[a, -a / 3]], np.float32))
        t = float(np.float32(a) / np.float32(127))
        if t > 65504:
            want = 65504.0
        else:
            d = np.abs(all16 - t)
            best = np.flatnonzero(d == d.min())
            if len(best) > 1:                 # tie: even significand
                best = [b for b in best if b % 2 == 0]
            want = all16[best[0]]
            if t >= 65520:
                want = 65504.0
        assert float(np.uint16(sb[0]).view(np.float16)) == want


def test_reconstruction_bound():
    """|x - code*s| <= max(s/2, a - qmax*s) for every element."""
    rng = np.random.default_rng(9)
    for qmax, fn, d in ((127, codec.quantize_k, 128), (7, codec.quantize_v, 128)):
        x = _rand_rows(rng, 300, d)
        codes, sb = fn(x)
        if qmax == 7:
            s = np.repeat(sb.view(np.float16).astype(np.float64), 32, axis=-1)
            a = np.repeat(np.max(np.abs(x.reshape(-1, 4, 32)), axis=-1).astype(np.float64), 32, axis=-1)
        else:
            s = np.repeat(sb.view(np.float16).astype(np.float64)[:, None], d, axis=-1)
            a = np.repeat(np.max(np.abs(x), axis=-1).astype(np.float64)[:, None], d, axis=-1)
        err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s)
        bound = np.maximum(s / 2, a - qmax * s)
        bound = np.where(s == 0, a, bound)
        assert np.all(err <= bound * (1 + 1e-12) + 0.0)
        normal = (s >= 2.0 ** -14) & (s < 65504)
        assert np.all(err[normal] <= s[normal] / 2 * (1 + 1e-12))


def test_code_ranges():
    rng = np.random.default_rng(3)
    x = _rand_rows(rng, 100, 128)
    kc, _ = codec.quantize_k(x)
    vc, _ = codec.quantize_v(x)
    assert kc.min() >= -127 and kc.max() <= 127
    assert vc.min() >= -7 and vc.max() <= 7


def test_v_nibble_layout_and_roundtrip():
    """Byte j of dimension row d holds slot 2j (low nibble) and slot 2j+1
    (high nibble) as two's complement; reading back gives the codes."""
    cache = codec.PagedCache(num_pages=2, num_kv_heads=1, head_dim=64)
    v = np.zeros((16, 1, 64), np.float32)
    k = np.zeros((16, 1, 64), np.float32)
    # group 0 of dim 0: slot 0 -> -1, slot 1 -> 3 (absmax 7 in the group via dim 1)
    v[:, 0, 1] = 7.0
    v[0, 0, 0] = -1.0
    v[1, 0, 0] = 3.0
    v[2, 0, 0] = -7.0
    v[3, 0, 0] = 7.0
    cache.write_tokens(np.full(16, 1), np.arange(16), k, v)
    row0 = cache.v_codes[1, 0, 0]
    assert row0[0] == 0x3F          # low nibble -1 (0xF), high nibble 3
    assert row0[1] == 0x79          # low nibble -7 (0x9), high nibble 7
    assert np.all(cache.v_codes[1, 0, 1] == 0x77)
    got = cache.v_codes_at(np.full(16, 1), np.arange(16), 0)
    assert got[0, 0] == -1 and got[1, 0] == 3 and got[2, 0] == -7 and got[3, 0] == 7
    # writing the odd slot later keeps the even nibble
    cache2 = codec.PagedCache(num_pages=1, num_kv_heads=1, head_dim=64)
    cache2.write_tokens(np.array([0]), np.array([4]), k[:1], v[:1])
    cache2.write_tokens(np.array([0]), np.array([5]), k[1:2], v[1:2])
    assert cache2.v_codes[0, 0, 0, 2] == 0x3F


def test_bf16_widening_exact():
    import torch
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(codec.bf16_bits_to_f32(bits), want)


def test_near_tie_codes_use_true_division():
    """Elements placed within a few ulps of code + 1/2: the codes must follow
    fp32 x/s exactly (a multiply by the reciprocal or a different rounding
    gives different codes on some of them)."""
    rng = np.random.default_rng(21)
    n_checked = 0
    for _ in range(400):
        s = np.float32(np.float16(rng.uniform(0.01, 3.0)))
        k = int(rng.integers(-126, 126))
        t = np.float32((k + 0.5) * float(s))
        xs = [t]
        for _ in range(3):
            xs.append(np.nextafter(xs[-1], np.float32(np.inf), dtype=np.float32))
        lo = [t]
        for _ in range(3):
            lo.append(np.nextafter(lo[-1], np.float32(-np.inf), dtype=np.float32))
        row = np.zeros(128, np.float32)
        row[0] = np.float32(127) * s          # pins the scale to s exactly
        vals = np.array(xs + lo[1:], np.float32)
        row[1: 1 + len(vals)] = vals
        codes, sb = codec.quantize_k(row[None])
        assert Fraction(float(np.uint16(sb[0]).view(np.float16))) == Fraction(float(s))
        for j, x in enumerate(vals):
            assert int(codes[0, 1 + j]) == exact_fp.codec_code(float(x), Fraction(float(s)), 127)
            n_checked += 1
    assert n_checked > 2000


def test_scale_is_single_rounding_of_exact_quotient():
    """fp16(fp32(a/q)) never double-rounds for q = 127 or 7: an fp32 a other
    than q*t sits at least 2^6 (resp. 2^2) fp32 ulps of t away from q*t, so
    the fp32 quotient cannot land on an fp16 half-way point t unless the exact
    quotient is t.  The scale therefore equals the fp16 rounding of the exact
    quotient; checked on values built around fp16 half-way points."""
    rng = np.random.default_rng(22)
    for qmax in (127, 7):
        for _ in range(1500):
            e = int(rng.integers(-10, 12))
            m = int(rng.integers(1024, 2047))
            t = (m + 0.5) * 2.0 ** (e - 10)             # fp16 half-way point
            a = np.float32(qmax * t)
            for step in range(-2, 3):
                aa = a
                for _ in range(abs(step)):
                    aa = np.nextafter(aa, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
                _, sb = codec.quantize_block(np.array([[aa, 0.0]], np.float32), qmax)
                direct = exact_fp.rne_f16(Fraction(float(aa)) / qmax)
                direct = Fraction(65504) if direct == exact_fp.INF else direct
                assert Fraction(float(np.uint16(sb[0]).view(np.float16))) == direct
