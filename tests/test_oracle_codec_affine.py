"""Pins for the oracle's affine codec variant (CPU only).

The affine reading (unsigned codes with a zero point, range widened to
include zero, fp16 scale; blog.123qwe.co.kr/?p=3927 section 5 names the codec
affine) is checked against hand-derived golden cases, a closed form, an
independent exact-rational evaluation of every rounding step, the
reconstruction bound, the stored byte layout, and -- for attention over an
affine cache -- textbook softmax attention on exactly representable inputs.
"""

import json
import os

import numpy as np
import pytest

from oracle import attention, codec
from tests import exact_fp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_affine_cases.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden_cases(case):
    if case["kind"] == "k":
        x = np.zeros(64, np.float32)
        x[: len(case["x"])] = case["x"]
        c, z, s = codec.quantize_k_affine(x[None])
        assert list(c[0, : len(case["x"])]) == case["codes"]
        assert np.all(c[0, len(case["x"]):] == case["zero"])      # padding encodes zero
        assert int(z[0]) == case["zero"]
        assert int(s[0]) == int(case["scale_bits"], 16)
    else:
        groups, codes = case["x_groups"], case["codes_groups"]
        x = np.zeros(64, np.float32)
        for g, row in enumerate(groups):
            x[32 * g: 32 * g + len(row)] = row
        c, z, s = codec.quantize_v_affine(x[None])
        for g, exp in enumerate(codes):
            assert list(c[0, 32 * g: 32 * g + len(exp)]) == exp
            assert int(z[0, g]) == case["zeros"][g]
            assert int(s[0, g]) == int(case["scale_bits"][g], 16)


def test_lossless_closed_form():
    """x = (c - z) * s with fp16 s, codes that reach 0 and qmax: scale, zero
    point and codes come back exactly."""
    rng = np.random.default_rng(21)
    for qmax, fn, D in ((255, codec.quantize_k_affine, 128), (15, codec.quantize_v_affine, 32)):
        for _ in range(300):
            e = int(rng.integers(-12, 8))
            s = np.float32(np.float16(int(rng.integers(1024, 2048)) * 2.0 ** (e - 10)))
            z = int(rng.integers(0, qmax + 1))
            c = rng.integers(0, qmax + 1, size=D)
            c[0], c[1] = 0, qmax
            x = ((c - z).astype(np.float32) * s).astype(np.float32)
            codes, zz, sb = fn(x[None])
            assert np.array_equal(codes[0], c.astype(np.uint8))
            assert int(np.asarray(zz).ravel()[0]) == z
            assert int(np.asarray(sb).ravel()[0]) == int(np.float16(s).view(np.uint16))


def _rows(rng, n, d):
    out = []
    for _ in range(n):
        mag = 10.0 ** rng.uniform(-6, 5)
        r = (rng.standard_normal(d) * mag + rng.uniform(-2, 2) * mag).astype(np.float32)
        if rng.random() < 0.2:
            r = np.abs(r)                    # one-signed blocks: lo or hi widened to 0
        if rng.random() < 0.1:
            r = -np.abs(r)
        out.append(r)
    return np.stack(out)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_matches_exact_rational_rounding(kind):
    rng = np.random.default_rng(22 if kind == "k" else 23)
    d, qmax = (64, 255) if kind == "k" else (32, 15)
    x = _rows(rng, 60, d)
    fn = codec.quantize_k_affine if kind == "k" else codec.quantize_v_affine
    codes, zeros, sb = fn(x)
    zeros, sb = np.asarray(zeros).reshape(60, -1)[:, 0], np.asarray(sb).reshape(60, -1)[:, 0]
    for i in range(x.shape[0]):
        lo, hi = min(float(np.min(x[i])), 0.0), max(float(np.max(x[i])), 0.0)
        s = exact_fp.affine_scale(lo, hi, qmax)
        assert exact_fp.Fraction(float(np.uint16(sb[i]).view(np.float16))) == s
        z = exact_fp.affine_zero(lo, s, qmax)
        assert int(zeros[i]) == z
        for j in range(d):
            assert int(codes[i, j]) == exact_fp.affine_code(float(x[i, j]), s, z, qmax)


def test_reconstruction_bound():
    """With a normal fp16 scale: |x - (c - z) s| <= s * (1.5 + qmax * 2^-10),
    and <= s/2 for every element the clamp leaves alone."""
    rng = np.random.default_rng(24)
    for qmax, fn, d in ((255, codec.quantize_k_affine, 128), (15, codec.quantize_v_affine, 128)):
        x = _rows(rng, 300, d)
        codes, zeros, sb = fn(x)
        if qmax == 15:
            xh = codec.dequantize_v_affine(codes, zeros, sb)
            s = np.repeat(sb.view(np.float16).astype(np.float64), 32, axis=-1)
        else:
            xh = codec.dequantize_k_affine(codes, zeros, sb)
            s = np.repeat(sb.view(np.float16).astype(np.float64)[:, None], d, axis=-1)
        normal = s >= 2.0 ** -14
        err = np.abs(x.astype(np.float64) - xh)
        assert np.all(err[normal] <= s[normal] * (1.5 + qmax * 2.0 ** -10))
        inner = normal & (codes > 0) & (codes < qmax)
        assert np.all(err[inner] <= s[inner] / 2 * (1 + 1e-12))


def test_stored_bytes_and_dequant():
    """Key code byte = code XOR 0x80, key zero byte = z XOR 0x80, value
    nibbles unsigned; the cache dequantizes to (code - z) * s."""
    cache = codec.PagedCache(2, 1, 64, codec="affine")
    k = np.zeros((1, 1, 64), np.float32)
    k[0, 0, :3] = [-128.0, 127.0, 1.0]            # s 1, z 128 -> codes 0, 255, 129
    v = np.zeros((1, 1, 64), np.float32)
    v[0, 0, :3] = [-8.0, 7.0, 2.0]                # group 0: s 1, z 8 -> codes 0, 15, 10
    cache.write_tokens(np.array([1]), np.array([3]), k, v)
    assert list(cache.k_codes[1, 0, 3, :4].view(np.uint8)) == [0x80, 0x7F, 0x01, 0x00]
    assert int(cache.k_zeros[1, 0, 3].view(np.uint8)) == 0x00     # 128 ^ 0x80
    assert int(cache.k_scales[1, 0, 3]) == 0x3C00
    # slot 3 is the high nibble of byte 1
    assert [int(cache.v_codes[1, 0, d, 1] >> 4) for d in range(3)] == [0, 15, 10]
    assert list(cache.v_zeros[1, 0, 3]) == [8, 0]
    kh, vh = cache.dequant_tokens(np.array([1]), np.array([3]), 0)
    assert np.array_equal(kh[0, :3], [-128.0, 127.0, 1.0]) and np.all(kh[0, 3:] == 0)
    assert np.array_equal(vh[0, :3], [-8.0, 7.0, 2.0]) and np.all(vh[0, 3:] == 0)


def test_attention_lossless_affine_cache_is_textbook_attention():
    """Inputs exactly representable by the affine codec: the oracle's decode
    over the affine cache equals textbook softmax attention on the raw
    inputs (float64)."""
    rng = np.random.default_rng(25)
    T, H, D, Hq = 40, 2, 64, 4
    s_k, s_v = np.float32(0.0625), np.float32(0.5)
    ck = rng.integers(0, 256, size=(T, H, D)); zk = rng.integers(60, 200, size=(T, H))
    ck[:, :, 0], ck[:, :, 1] = 0, 255
    k = ((ck - zk[..., None]) * s_k).astype(np.float32)
    cv = rng.integers(0, 16, size=(T, H, D)); zv = rng.integers(3, 12, size=(T, H, D // 32))
    cv[:, :, ::32], cv[:, :, 1::32] = 0, 15
    v = ((cv - np.repeat(zv, 32, axis=-1)) * s_v).astype(np.float32)
    cache = codec.PagedCache(4, H, D, codec="affine")
    pt = np.array([[2, 0, 3]], np.int32)
    codec.append(cache, k, v, "f32", np.array([0, T]), np.array([0]), pt)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    scale = 0.125
    got = attention.decode(cache, q, "f32", pt, np.array([T]), scale)
    G = Hq // H
    for h in range(Hq):
        sc = (k[:, h // G, :].astype(np.float64) @ q[0, h].astype(np.float64)) * scale
        w = np.exp(sc - sc.max())
        want = (w[:, None] * v[:, h // G, :].astype(np.float64)).sum(0) / w.sum()
        assert np.max(np.abs(got[0, h] - want)) <= 1e-12
