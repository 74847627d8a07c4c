"""GPU parity of the affine codec variant (blog.123qwe.co.kr/?p=3927,
section 5 names the k8v4 codec affine): kv_quant_append codes, zero points
and scales bit-exact with the oracle (ragged batches with odd start slots,
edge rows: zeros, one-signed rows, ties, tiny and huge magnitudes), and
decode, verify and shared-prefix decode over an affine cache against the
fp64 oracle on the kernels that support it (variants 4 and 5)."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache
from oracle import attention

pytestmark = pytest.mark.gpu


def _assert_same(got, ref):
    for name in ("k_codes", "k_scales", "k_zeros", "v_codes", "v_scales", "v_zeros"):
        assert np.array_equal(got[name], getattr(ref, name)), f"{name} differ"


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32"), (128, "f32"), (64, "bf16")])
def test_append_bit_exact(D, dtype):
    from tests.gpu_util import cache_to_host, upload_cache
    from tests.test_gpu_append import _resplit
    rng = np.random.default_rng(D + 7 * len(dtype))
    w = workloads.build("aff_append", seed=71, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                        seq_lens=[1, 15, 16, 17, 33, 250, 0, 61], outliers=True, spare_pages=3)
    w = _resplit(w, rng)
    print(f"[affine] append D {D} {dtype}", flush=True)
    _assert_same(cache_to_host(upload_cache(w, codec="affine")), oracle_cache(w, codec_name="affine"))


def test_append_bulk_prompt_bit_exact():
    """A 4096-token prompt from position 0 in one call: every chunk of 16 new
    tokens fills one page (the page-block path)."""
    from tests.gpu_util import cache_to_host, upload_cache
    w = workloads.gqa_decode_4k()
    _assert_same(cache_to_host(upload_cache(w, codec="affine")), oracle_cache(w, codec_name="affine"))


def test_append_edge_rows():
    """Rows that stress the rule: all zero, one-signed (lo or hi widened to
    zero), constant, exact ties, tiny (subnormal or zero scale) and huge
    (saturating scale) magnitudes, one large element among small ones."""
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import cache_to_host, to_dev
    from oracle import codec
    D, H = 128, 1
    rows = []
    base = np.linspace(-1, 1, D).astype(np.float32)
    rows += [np.zeros(D), np.abs(base) + 0.5, -np.abs(base) - 0.25, np.full(D, 3.0), np.full(D, -2.5)]
    ties = np.zeros(D, np.float32); ties[:8] = [-128, 127, 1.5, 2.5, -0.5, -1.5, 0.5, 3.5]
    rows.append(ties)
    rows += [base * 1e-7, base * 1e-9, base * 3e-6, base * 1e30, base * 7e4]
    spike = base * 1e-3; spike[17] = 50.0
    rows.append(spike)
    x = np.stack([r.astype(np.float32) for r in rows])[:, None, :]         # [N][1][D]
    N = x.shape[0]
    pages = (N + 15) // 16
    pt = np.arange(pages, dtype=np.int32)[None]
    cache = q8.PagedKVCache(pages, H, D, codec="affine")
    q8.kv_quant_append(cache, to_dev(x), to_dev(x[::-1].copy()), to_dev(np.array([0, N], np.int32)),
                       to_dev(np.array([0], np.int32)), to_dev(pt))
    torch.cuda.synchronize()
    ref = codec.PagedCache(pages, H, D, codec="affine")
    codec.append(ref, x, x[::-1].copy(), "f32", np.array([0, N]), np.array([0]), pt)
    _assert_same(cache_to_host(cache), ref)


DECODE_CFGS = [None, dict(variant=4, waves_per_wg=8), dict(variant=5), dict(variant=5, waves_per_wg=8)]


def _attend(w, cache, cfg, n_pref=0):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev
    c = None if cfg is None else q8.make_config(**cfg)
    q, lens, pt = to_dev(w.q, w.dtype), to_dev(w.seq_lens), to_dev(w.page_table)
    msl = int(w.seq_lens.max())
    if w.n_draft:
        out = q8.attn_verify_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=c)
    elif n_pref:
        out = q8.attn_decode_prefix_q8k4v(cache, q, lens, msl, pt, n_pref, w.softmax_scale, cfg=c)
    else:
        out = q8.attn_decode_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=c)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _want(w, oc):
    f = attention.verify if w.n_draft else attention.decode
    return f(oc, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)


@pytest.mark.parametrize("hq,hkv,D,dt", [(32, 8, 128, "bf16"), (8, 8, 64, "f32"), (16, 2, 128, "bf16"),
                                         (16, 8, 64, "bf16")], ids=str)
def test_decode_parity(hq, hkv, D, dt):
    from tests.gpu_util import upload_cache
    w = workloads.build("aff_dec", seed=72 + hq + D, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=dt,
                        seq_lens=[2000, 333, 17, 0], outliers=True)
    cache, oc = upload_cache(w, codec="affine"), oracle_cache(w, codec_name="affine")
    want = _want(w, oc)
    for cfg in DECODE_CFGS:
        err = normalized_err(w, _attend(w, cache, cfg), want)
        print(f"[affine] decode Hq {hq} Hkv {hkv} D {D} cfg {cfg}: {err:.3e}", flush=True)
        assert err <= ATOL_SIGMA, (cfg, err)


@pytest.mark.parametrize("nd", [2, 3, 8])
def test_verify_parity(nd):
    from tests.gpu_util import upload_cache
    w = workloads.build("aff_ver", seed=80 + nd, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1500, 200 + nd], n_draft=nd, outliers=True)
    cache, oc = upload_cache(w, codec="affine"), oracle_cache(w, codec_name="affine")
    want = _want(w, oc)
    for cfg in (None, dict(variant=5, waves_per_wg=4)):
        err = normalized_err(w, _attend(w, cache, cfg), want)
        print(f"[affine] verify W {nd} cfg {cfg}: {err:.3e}", flush=True)
        assert err <= ATOL_SIGMA, (cfg, err)


def test_shared_prefix_parity():
    from tests.gpu_util import upload_cache
    w = workloads.multi_session(seed=85, sessions=5, prefix=512, max_suffix=700)
    cache, oc = upload_cache(w, codec="affine"), oracle_cache(w, codec_name="affine")
    want = _want(w, oc)
    err = normalized_err(w, _attend(w, cache, None, n_pref=w.shared_prefix // 16), want)
    print(f"[affine] cascade: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, err


@pytest.mark.slow
def test_full_64k_decode_affine():
    from tests.gpu_util import upload_cache
    w = workloads.gqa_decode_64k()
    err = normalized_err(w, _attend(w, upload_cache(w, codec="affine"), None),
                         _want(w, oracle_cache(w, codec_name="affine")))
    print(f"[affine] 64K decode: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, err
