"""GPU parity with queries of wide dynamic range.

The kernels feed the query to the int8 MFMA as a 23-bit fixed-point number
per row (three int8 digits, one exponent per row): an element loses bits only
when it lies more than 2^15 below its row's largest magnitude, by at most
2^-22 of that maximum.  These cases stress that rounding against the fp64
oracle (exact softmax attention over the dequantized cache, the decode unit of
blog.123qwe.co.kr/?p=3927, section 5): 1 % of the query channels scaled by 8,
64 or 1024, and queries whose elements spread over six decades, in bf16 and
fp32, on both kernels, verify, the shared-prefix cascade and the one-call
decode step.  Tolerance: 2e-3 per sigma-normalised element, as everywhere."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[query range] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert err <= ATOL_SIGMA, (label, err)


DECODE = [dict(q_outlier=8), dict(q_outlier=64), dict(q_outlier=1024), dict(q_decades=6)]


@pytest.mark.parametrize("rng", DECODE, ids=str)
@pytest.mark.parametrize("cfg", [None, dict(variant=5), dict(fused_combine=1)], ids=str)
def test_decode_outlier_and_wide_queries_bf16(rng, cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("qr_decode", seed=301, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[2000, 777], outliers=True, **rng)
    cache = upload_cache(w)
    c = None if cfg is None else q8.make_config(**cfg)
    _check(w, run_attention(w, cache, cfg=c), oracle_out(w), f"decode bf16 {rng} cfg {cfg}")


@pytest.mark.parametrize("shape", [(2, 1, 64, 256), (8, 2, 128, 1500)], ids=str)
@pytest.mark.parametrize("rng", [dict(q_decades=6), dict(q_outlier=1024)], ids=str)
@pytest.mark.parametrize("cfg", [None, dict(variant=5)], ids=str)
def test_decode_wide_queries_fp32(shape, rng, cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    hq, hkv, D, L = shape
    w = workloads.build("qr_f32", seed=302, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype="f32",
                        seq_lens=[L], outliers=True, **rng)
    cache = upload_cache(w)
    c = None if cfg is None else q8.make_config(**cfg)
    _check(w, run_attention(w, cache, cfg=c), oracle_out(w), f"decode fp32 {shape} {rng} cfg {cfg}")


@pytest.mark.parametrize("n_draft", [4, 8])
@pytest.mark.parametrize("rng", [dict(q_outlier=1024), dict(q_decades=6)], ids=str)
def test_verify_outlier_and_wide_queries(n_draft, rng):
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("qr_verify", seed=303 + n_draft, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        dtype="bf16", seq_lens=[1800 + n_draft, 300 + n_draft], n_draft=n_draft, outliers=True,
                        **rng)
    cache = upload_cache(w)
    _check(w, run_attention(w, cache), oracle_out(w), f"verify W {n_draft} {rng}")


@pytest.mark.parametrize("rng", [dict(q_outlier=1024), dict(q_decades=6)], ids=str)
def test_cascade_outlier_and_wide_queries(rng):
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.build("qr_cascade", seed=304, num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=[1024 + 300, 1024 + 17, 1024, 1024 + 900], outliers=True, shared_prefix=1024,
                        **rng)
    cache = upload_cache(w)
    _check(w, run_prefix(w, cache, 1024 // 16), oracle_out(w), f"cascade {rng}")


@pytest.mark.parametrize("rng", [dict(q_outlier=1024), dict(q_decades=6)], ids=str)
def test_decode_step_outlier_and_wide_queries(rng):
    """attn_decode_append_q8k4v (append the step's token and attend, one
    launch) with the same queries: codes bit-exact, output in tolerance."""
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import cache_to_host, to_dev
    w = workloads.build("qr_step", seed=305, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1333, 64], outliers=True, **rng)
    a = w.appends[-1]
    rows = (a.cu_new[1:] - 1).astype(np.int64)
    keep = np.setdiff1d(np.arange(a.cu_new[-1]), rows)
    cache = q8.PagedKVCache(w.num_pages, w.num_kv_heads, w.head_dim)
    q8.kv_quant_append(cache, to_dev(a.k[keep], "bf16"), to_dev(a.v[keep], "bf16"),
                       to_dev(np.concatenate([[0], np.cumsum(np.diff(a.cu_new) - 1)]).astype(np.int32)),
                       to_dev(a.start_pos), to_dev(a.page_table))
    got = q8.attn_decode_append_q8k4v(cache, to_dev(a.k[rows], "bf16"), to_dev(a.v[rows], "bf16"),
                                      to_dev(w.q, "bf16"), to_dev(w.seq_lens), int(w.seq_lens.max()),
                                      to_dev(w.page_table))
    torch.cuda.synchronize()
    oc = oracle_cache(w)
    host = cache_to_host(cache)
    assert np.array_equal(host["k_codes"], oc.k_codes) and np.array_equal(host["v_codes"], oc.v_codes)
    assert np.array_equal(host["k_scales"], oc.k_scales) and np.array_equal(host["v_scales"], oc.v_scales)
    _check(w, got.cpu().numpy().astype(np.float64), oracle_out(w, oc), f"decode step {rng}")
