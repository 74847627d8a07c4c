"""GPU parity of attn_decode_q8k4v against the fp64 oracle: the named
workloads, ragged batches (empty, partial-page, multi-page sequences), every
group size, every launch-shape configuration the tuner may choose, split and
page-permutation invariance, determinism, and the full 64K workload."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu

CONFIGS = [None,
           dict(split_pages=1), dict(split_pages=3, waves_per_wg=2), dict(wgs_per_cu=8),
           dict(wgs_per_cu=1, fused_combine=0), dict(wgs_per_cu=3, fused_combine=1),
           dict(variant=4, stages=2), dict(variant=4, waves_per_wg=2, stages=3), dict(variant=4, fused_combine=1),
           dict(variant=4, waves_per_wg=8, stages=3, fused_combine=1),
           dict(variant=4, split_pages=5, waves_per_wg=2, stages=2), dict(variant=5), dict(variant=5, fused_combine=1),
           dict(variant=5, waves_per_wg=2, stages=3), dict(variant=5, waves_per_wg=8)]


def _cfg(d):
    import decode_attention_quantized_kv_amd as q8
    return None if d is None else q8.make_config(**d)


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[decode] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (label, err)
    return err


@pytest.mark.parametrize("name", ["tiny_decode_256", "gqa_decode_4096"])
def test_named_workloads(name):
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.NAMED[name]()
    cache = upload_cache(w)
    want = oracle_out(w)
    _check(w, run_attention(w, cache), want, name)


@pytest.mark.parametrize("hq,hkv,D,dtype", [(32, 8, 128, "bf16"), (8, 4, 64, "f32"), (8, 8, 128, "bf16"),
                                             (32, 4, 128, "bf16"), (16, 8, 64, "bf16"), (4, 1, 128, "f32")])
def test_ragged_batch_all_groups(hq, hkv, D, dtype):
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("ragged", seed=hq + hkv + D, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=dtype,
                        seq_lens=[1, 15, 16, 17, 0, 300, 1000, 47], outliers=True)
    cache = upload_cache(w)
    want = oracle_out(w)
    got = run_attention(w, cache)
    _check(w, got, want, f"ragged hq={hq} hkv={hkv} D={D} {dtype}")
    assert np.all(got[4] == 0)


def test_many_sequences():
    """48 ragged sequences (lengths 0..1200, seeded): the splits of every
    sequence are dealt over the XCDs starting at a different one per
    sequence, and empty sequences give zero rows."""
    from tests.gpu_util import run_attention, upload_cache
    lens = np.random.default_rng(2024).integers(0, 1201, size=48)
    lens[[5, 17]] = 0
    w = workloads.build("many", seed=31, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=lens.tolist(), outliers=True)
    cache = upload_cache(w)
    got = run_attention(w, cache)
    _check(w, got, oracle_out(w), "48 sequences")
    assert np.all(got[5] == 0) and np.all(got[17] == 0)


@pytest.mark.parametrize("hq,hkv,D,fp32", [(32, 8, 128, False), (2, 1, 64, True)])
def test_every_sequence_empty(hq, hkv, D, fp32):
    """Degenerate batch: every sequence is empty (max_seq_len 0).  The plan
    has one split, no page is read, and every output row is written as zero
    over an output buffer that starts as NaN."""
    import torch

    import decode_attention_quantized_kv_amd as q8
    cache = q8.PagedKVCache(1, hkv, D)
    q = torch.randn(3, hq, D, device="cuda")
    if not fp32:
        q = q.to(torch.bfloat16)
    lens = torch.zeros(3, dtype=torch.int32, device="cuda")
    table = torch.zeros(3, 1, dtype=torch.int32, device="cuda")
    out = torch.full((3, hq, D), float("nan"), device="cuda")
    q8.attn_decode_q8k4v(cache, q, lens, 0, table, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0), (hq, hkv, D)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "default" if c is None else "-".join(f"{k}{v}" for k, v in c.items()))
def test_every_launch_configuration(cfg):
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("cfg", seed=77, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[2000, 37, 900], outliers=True)
    cache = upload_cache(w)
    _check(w, run_attention(w, cache, cfg=_cfg(cfg)), oracle_out(w), f"cfg {cfg}")


def test_permuted_pool_and_determinism():
    from tests.gpu_util import run_attention, upload_cache
    kw = dict(seed=5, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seq_lens=[777, 64],
              outliers=True)
    a = workloads.build("a", permute_pages=False, **kw)
    b = workloads.build("b", permute_pages=True, **kw)
    ca, cb = upload_cache(a), upload_cache(b)
    ga, gb = run_attention(a, ca), run_attention(b, cb)
    assert np.array_equal(ga, gb)                        # physical placement is invisible
    assert np.array_equal(ga, run_attention(a, ca))      # bit-identical reruns
    _check(a, ga, oracle_out(a), "permuted pool")


def test_value_magnitudes():
    """Tolerance holds relative to sigma for small and large value scales."""
    from tests.gpu_util import run_attention, upload_cache
    for vs in (1e-2, 1e2):
        w = workloads.build("vs", seed=9, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                            seq_lens=[1500], outliers=True, value_scale=vs)
        _check(w, run_attention(w, upload_cache(w)), oracle_out(w), f"value scale {vs}")


@pytest.mark.slow
def test_full_64k_decode():
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.gqa_decode_64k()
    cache = upload_cache(w)
    ocache = oracle_cache(w)
    want = oracle_out(w, ocache)
    _check(w, run_attention(w, cache), want, "gqa_decode_65536")
