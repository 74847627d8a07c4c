"""GPU parity for softmax scales the ABI accepts but the workloads never use
(zero: uniform weights; negative: the ordering of the scores reversed; large:
a near one-hot softmax), on decode and verify with every kernel, and for
contexts of 128K and 200K tokens (split counts and page walks past the 64K
configuration), against the fp64 oracle."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache
from oracle import attention

pytestmark = pytest.mark.gpu

DECODE_CFGS = [None, dict(variant=5), dict(variant=4, waves_per_wg=8), dict(fused_combine=1)]
VERIFY_CFGS = [None, dict(variant=5, waves_per_wg=4), dict(fused_combine=1)]


def _run(w, cache, scale, cfg):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev
    c = None if cfg is None else q8.make_config(**cfg)
    q, lens, pt = to_dev(w.q, w.dtype), to_dev(w.seq_lens), to_dev(w.page_table)
    msl = int(w.seq_lens.max())
    if w.n_draft:
        out = q8.attn_verify_q8k4v(cache, q, lens, msl, pt, scale, cfg=c)
    else:
        out = q8.attn_decode_q8k4v(cache, q, lens, msl, pt, scale, cfg=c)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _oracle(w, oc, scale):
    f = attention.verify if w.n_draft else attention.decode
    return f(oc, w.q, w.dtype, w.page_table, w.seq_lens, scale)


@pytest.mark.parametrize("scale", [0.0, -0.0883883, 0.7], ids=["zero", "negative", "large"])
def test_decode_softmax_scales(scale):
    from tests.gpu_util import upload_cache
    w = workloads.build("scale_dec", seed=61, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=[1500, 333, 64], outliers=True)
    cache, oc = upload_cache(w), oracle_cache(w)
    want = _oracle(w, oc, scale)
    for cfg in DECODE_CFGS:
        err = normalized_err(w, _run(w, cache, scale, cfg), want)
        print(f"[scale] decode scale {scale} cfg {cfg}: {err:.3e}", flush=True)
        assert err <= ATOL_SIGMA, (scale, cfg, err)


@pytest.mark.parametrize("scale", [0.0, -0.0883883, 0.7], ids=["zero", "negative", "large"])
def test_verify_softmax_scales(scale):
    from tests.gpu_util import upload_cache
    w = workloads.build("scale_ver", seed=62, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=[900, 200], n_draft=5, outliers=True)
    cache, oc = upload_cache(w), oracle_cache(w)
    want = _oracle(w, oc, scale)
    for cfg in VERIFY_CFGS:
        err = normalized_err(w, _run(w, cache, scale, cfg), want)
        print(f"[scale] verify scale {scale} cfg {cfg}: {err:.3e}", flush=True)
        assert err <= ATOL_SIGMA, (scale, cfg, err)


@pytest.mark.slow
@pytest.mark.parametrize("ctx,nd", [(131072, 0), (131072, 8), (200000, 0), (200000, 8)])
def test_long_context_decode_and_verify(ctx, nd):
    from tests.gpu_util import upload_cache
    w = workloads.build(f"long_{ctx}_{nd}", seed=63 + nd, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        dtype="bf16", seq_lens=[ctx + nd], n_draft=nd, outliers=True)
    cache = upload_cache(w)
    want = _oracle(w, oracle_cache(w), w.softmax_scale)
    err = normalized_err(w, _run(w, cache, w.softmax_scale, None), want)
    print(f"[long] ctx {ctx} n_draft {nd}: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (ctx, nd, err)
