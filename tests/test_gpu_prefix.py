"""GPU parity of attn_decode_prefix_q8k4v, the shared-prefix cascade for
concurrent sessions over one cached prompt prefix (blog.123qwe.co.kr/?p=3927,
section 5): ragged sessions against the fp64 oracle with every suffix
kernel, suffixes that are empty, one token or a partial page, group sizes
1..8 and D 64, many sessions (several row chunks in the prefix block), a
prefix shorter than the shared part, agreement with the plain decode entry
point, and the full 16-session workload (32768-token shared prefix)."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[prefix] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert err <= ATOL_SIGMA, (label, err)


@pytest.mark.parametrize("cfg", [None, dict(variant=4, stages=2, waves_per_wg=2), dict(variant=4, stages=3),
                                 dict(variant=5), dict(variant=5, waves_per_wg=8), dict(fused_combine=1),
                                 dict(wgs_per_cu=3)], ids=str)
def test_ragged_sessions_every_suffix_kernel(cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.multi_session(seed=21, sessions=6, prefix=256, max_suffix=700)
    c = None if cfg is None else q8.make_config(**cfg)
    _check(w, run_prefix(w, upload_cache(w), w.shared_prefix // 16, cfg=c), oracle_out(w), f"6 sessions cfg {cfg}")


def test_empty_one_token_and_partial_page_suffixes():
    from tests.gpu_util import run_prefix, upload_cache
    P = 320
    w = workloads.build("prefix_edges", seed=22, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=[P, P + 1, P + 16, P + 17, P + 500, P], shared_prefix=P, outliers=True)
    _check(w, run_prefix(w, upload_cache(w), P // 16), oracle_out(w), "edge suffixes")


def test_prefix_only_sessions():
    """Every session is exactly the prefix: the suffix pass has no pages."""
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.build("prefix_only", seed=23, num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=[512] * 5, shared_prefix=512)
    _check(w, run_prefix(w, upload_cache(w), 32), oracle_out(w), "prefix only")


@pytest.mark.parametrize("hq,hkv,d,dt", [(8, 8, 64, "f32"), (8, 4, 64, "bf16"), (16, 4, 128, "f32"),
                                         (32, 4, 128, "bf16"), (16, 2, 64, "bf16")], ids=str)
def test_group_sizes_and_head_dims(hq, hkv, d, dt):
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.build(f"prefix_g{hq // hkv}_d{d}", seed=24 + hq + d, num_q_heads=hq, num_kv_heads=hkv,
                        head_dim=d, dtype=dt, seq_lens=[400, 273, 1000], shared_prefix=256, outliers=True)
    _check(w, run_prefix(w, upload_cache(w), 16), oracle_out(w), f"Hq {hq} Hkv {hkv} D {d} {dt}")


def test_many_sessions_several_row_chunks():
    """40 sessions x group 4 = 160 prefix rows per kv head (five 32-row chunks)."""
    from tests.gpu_util import run_prefix, upload_cache
    rng = np.random.default_rng(25)
    lens = 512 + rng.integers(0, 200, size=40)
    w = workloads.build("prefix_40", seed=25, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=lens, shared_prefix=512, outliers=True)
    _check(w, run_prefix(w, upload_cache(w), 32), oracle_out(w), "40 sessions")


def test_single_session():
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.build("prefix_1", seed=26, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[3000], shared_prefix=2048, outliers=True)
    _check(w, run_prefix(w, upload_cache(w), 128), oracle_out(w), "1 session")


def test_prefix_shorter_than_shared_part():
    """Declaring fewer shared pages than the sessions really share is valid:
    the rest is read per session."""
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.multi_session(seed=27, sessions=4, prefix=512, max_suffix=300)
    cache = upload_cache(w)
    want = oracle_out(w)
    for n_pref in (1, 7, 31):
        _check(w, run_prefix(w, cache, n_pref), want, f"n_prefix_pages {n_pref}")


def test_zero_prefix_is_the_plain_decode_and_cascade_agrees_with_it():
    from tests.gpu_util import run_attention, run_prefix, upload_cache
    w = workloads.multi_session(seed=28, sessions=5, prefix=1024, max_suffix=900)
    cache = upload_cache(w)
    plain = run_attention(w, cache)
    assert np.array_equal(run_prefix(w, cache, 0), plain)
    casc = run_prefix(w, cache, 64)
    _check(w, casc, plain, "cascade vs plain decode")
    _check(w, casc, oracle_out(w), "cascade vs oracle")


def test_repeated_calls_are_deterministic():
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.multi_session(seed=29, sessions=3, prefix=256, max_suffix=400)
    cache = upload_cache(w)
    a = run_prefix(w, cache, 16)
    b = run_prefix(w, cache, 16)
    assert np.array_equal(a, b)


@pytest.mark.slow
def test_full_multi_session_16x32768_cascade():
    from tests.gpu_util import run_prefix, upload_cache
    w = workloads.multi_session()
    _check(w, run_prefix(w, upload_cache(w), w.shared_prefix // 16), oracle_out(w), "multi_session_16x32768")
