"""Pins for the oracle's fp64 attention over the dequantized paged cache
(CPU only): closed forms, a textbook library implementation on lossless
inputs, brute force, causal/structural invariants and a rigorous error bound
against unquantized attention."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, codec
from tests.util import oracle_cache, oracle_out


def _lossless_rows(rng, n, d, qmax, group):
    """Rows x = code * s with power-of-two fp16 scales and one maximal code per
    scale group: the codec reproduces them exactly."""
    x = np.zeros((n, d), np.float32)
    for i in range(n):
        for g0 in range(0, d, group):
            s = 2.0 ** int(rng.integers(-6, 3))
            c = rng.integers(-qmax, qmax + 1, size=group)
            c[int(rng.integers(0, group))] = qmax
            x[i, g0:g0 + group] = c * s
    return x


def _cache_from_rows(k, v, d, permute=None):
    """Single sequence, one kv head, tokens in order, optional page permutation."""
    T = k.shape[0]
    npages = (T + 15) // 16
    perm = np.arange(npages) if permute is None else permute
    cache = codec.PagedCache(npages, 1, d)
    pos = np.arange(T)
    cache.write_tokens(perm[pos // 16], pos % 16, k[:, None, :], v[:, None, :])
    return cache, perm[None, :].astype(np.int32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("raw_scale", [None, 0.1])
def test_lossless_case_equals_library_softmax_attention(d, raw_scale):
    """The softmax scale is an fp32 argument: a value like 0.1 acts as
    fp32(0.1) widened, not as the decimal."""
    rng = np.random.default_rng(d)
    T = 200
    k = _lossless_rows(rng, T, d, 127, d)
    v = _lossless_rows(rng, T, d, 7, 32)
    cache, pt = _cache_from_rows(k, v, d, permute=rng.permutation((T + 15) // 16))
    q = rng.standard_normal((1, 3, d)).astype(np.float32)
    cache3 = codec.PagedCache(cache.num_pages, 3, d)     # 3 kv heads, same data
    for n in ("k_codes", "k_scales", "v_codes", "v_scales"):
        getattr(cache3, n)[:] = getattr(cache, n)[:, :1].repeat(3, axis=1)
    arg = float(np.float32(1 / math.sqrt(d))) if raw_scale is None else raw_scale
    scale = float(np.float32(arg))
    got = attention.decode(cache3, q, "f32", pt, np.array([T]), arg)
    # textbook attention on the raw (exactly representable) rows, by torch
    qt = torch.from_numpy(q.astype(np.float64))[0]
    kt = torch.from_numpy(k.astype(np.float64))
    vt = torch.from_numpy(v.astype(np.float64))
    ref = torch.softmax(scale * (qt @ kt.T), dim=-1) @ vt
    assert np.max(np.abs(got[0] - ref.numpy())) <= 1e-12


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    T, d = 77, 128
    k = np.tile(rng.standard_normal(d).astype(np.float32), (T, 1))
    v = rng.standard_normal((T, d)).astype(np.float32)
    cache, pt = _cache_from_rows(k, v, d)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    got = attention.decode(cache, q, "f32", pt, np.array([T]), 0.088)
    _, vh = attention.sequence_kv(cache, pt[0], T, 0)
    assert np.max(np.abs(got[0, 0] - vh.mean(axis=0))) <= 1e-12


def test_dominant_key_returns_its_value_row():
    rng = np.random.default_rng(2)
    T, d, j = 300, 64, 123
    k = (rng.standard_normal((T, d)) * 0.01).astype(np.float32)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, :] = 1.0
    k[j, :] = 2.0                    # score gap >= 2*64*c - small
    v = rng.standard_normal((T, d)).astype(np.float32)
    cache, pt = _cache_from_rows(k, v, d)
    c = 1.0
    got = attention.decode(cache, q, "f32", pt, np.array([T]), c)
    kh, vh = attention.sequence_kv(cache, pt[0], T, 0)
    s = c * (kh @ q[0, 0].astype(np.float64))
    gap = s[j] - np.max(np.delete(s, j))
    assert gap >= 40
    bound = 2 * T * math.exp(-gap) * np.max(np.abs(vh))
    assert np.max(np.abs(got[0, 0] - vh[j])) <= bound + 1e-15


def test_brute_force_scalar_loops():
    """Scalar triple loop with math.fsum/math.exp on a tiny GQA case."""
    w = workloads.build("bf", seed=17, num_q_heads=4, num_kv_heads=2, head_dim=64,
                        dtype="f32", seq_lens=[37, 5], outliers=False)
    cache = oracle_cache(w)
    got = oracle_out(w, cache)
    qf = w.q.astype(np.float64)
    c = float(np.float32(w.softmax_scale))
    for b in range(2):
        L = int(w.seq_lens[b])
        for h in range(4):
            kvh = h // 2
            rows = []
            for t in range(L):
                page = int(w.page_table[b, t // 16])
                slot = t % 16
                kc = cache.k_codes[page, kvh, slot].astype(int)
                ks = float(np.uint16(cache.k_scales[page, kvh, slot]).view(np.float16))
                byte = cache.v_codes[page, kvh, :, slot // 2].astype(int)
                nib = (byte >> 4) if slot % 2 else (byte & 0xF)
                vc = [n - 16 if n >= 8 else n for n in nib]
                vs = [float(np.uint16(x).view(np.float16)) for x in cache.v_scales[page, kvh, slot]]
                kk = [kc[dd] * ks for dd in range(64)]
                vv = [vc[dd] * vs[dd // 32] for dd in range(64)]
                rows.append((c * math.fsum(qf[b, h, dd] * kk[dd] for dd in range(64)), vv))
            m = max(r[0] for r in rows)
            ws = [math.exp(r[0] - m) for r in rows]
            den = math.fsum(ws)
            for dd in range(64):
                num = math.fsum(ws[t] * rows[t][1][dd] for t in range(L))
                assert abs(got[b, h, dd] - num / den) <= 1e-13 * max(1.0, abs(num / den))


def test_causal_verify_rows_equal_shorter_decodes():
    w = workloads.build("cv", seed=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        dtype="bf16", seq_lens=[133, 40], n_draft=5, outliers=True)
    cache = oracle_cache(w)
    ver = oracle_out(w, cache)
    for j in range(5):
        lens = w.seq_lens - 5 + j + 1
        dec = attention.decode(cache, w.q[:, j], "bf16", w.page_table, lens, w.softmax_scale)
        assert np.array_equal(ver[:, j], dec)


def test_page_permutation_and_shared_prefix_invariance():
    kw = dict(seed=8, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", outliers=True)
    a = workloads.build("a", seq_lens=[300], permute_pages=False, **kw)
    b = workloads.build("b", seq_lens=[300], permute_pages=True, **kw)
    assert not np.array_equal(a.page_table, b.page_table)
    assert np.array_equal(oracle_out(a), oracle_out(b))
    # sessions mapping one shared prefix == the same sessions with private copies
    sh = workloads.build("sh", seed=9, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16",
                         seq_lens=[64 + 3, 64 + 20, 64], shared_prefix=64)
    cache = oracle_cache(sh)
    out_shared = oracle_out(sh, cache)
    pre = sh.shared_prefix // 16
    priv_table = sh.page_table.copy()
    extra = codec.PagedCache(sh.num_pages + pre * 3, 2, 64)
    for n in ("k_codes", "k_scales", "v_codes", "v_scales"):
        getattr(extra, n)[: sh.num_pages] = getattr(cache, n)
    for s in range(3):
        new_ids = sh.num_pages + s * pre + np.arange(pre)
        for n in ("k_codes", "k_scales", "v_codes", "v_scales"):
            getattr(extra, n)[new_ids] = getattr(cache, n)[sh.page_table[s, :pre]]
        priv_table[s, :pre] = new_ids
    assert len(set(priv_table[:, :pre].ravel())) == 3 * pre
    out_priv = attention.decode(extra, sh.q, "bf16", priv_table, sh.seq_lens, sh.softmax_scale)
    assert np.array_equal(out_shared, out_priv)


@pytest.mark.parametrize("outliers", [False, True])
def test_bound_against_unquantized_attention(outliers):
    """|o_quant - o_exact|_d <= max_t |vhat - v|_{t,d} + (e^D - 1)(max_t v_d - min_t v_d)/2
    with D = max delta - min delta, delta_t the score change from quantizing K."""
    for seed in range(6):
        w = workloads.build("bd", seed=100 + seed, num_q_heads=4, num_kv_heads=1, head_dim=64,
                            dtype="f32", seq_lens=[512], outliers=outliers, permute_pages=False)
        cache = oracle_cache(w)
        got = oracle_out(w, cache)[0]
        a = w.appends[0]
        k = a.k[:, 0].astype(np.float64)
        v = a.v[:, 0].astype(np.float64)
        kh, vh = attention.sequence_kv(cache, w.page_table[0], 512, 0)
        c = float(np.float32(w.softmax_scale))
        for h in range(4):
            q = w.q[0, h].astype(np.float64)
            exact = attention.softmax_attention(q, k, v, c)
            delta = c * (kh @ q) - c * (k @ q)
            Dl = delta.max() - delta.min()
            bound = np.max(np.abs(vh - v), axis=0) + (math.exp(Dl) - 1) * (v.max(0) - v.min(0)) / 2
            assert np.all(np.abs(got[h] - exact) <= bound * (1 + 1e-9))


def test_zero_length_sequence_yields_zeros():
    w = workloads.build("z", seed=3, num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="f32",
                        seq_lens=[16, 0])
    out = oracle_out(w)
    assert np.all(out[1] == 0) and np.any(out[0] != 0)
