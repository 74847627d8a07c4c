"""GPU parity of attn_prefill_q8k4v, chunked-prefill attention over the
quantized cache (blog.123qwe.co.kr/?p=3927, section 3 weights 4k and 64k
prompt prefill in the service cost): a chunk of new tokens, appended in bulk,
attends the cached context and itself causally -- the verify computation at
chunk lengths up to 1024 -- against the fp64 oracle, for several chunk
lengths, group sizes, head sizes, ragged contexts, both codecs and launch
configurations."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache
from oracle import attention

pytestmark = pytest.mark.gpu


def _prefill(w, cache, cfg=None):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev
    c = None if cfg is None else q8.make_config(**cfg)
    out = q8.attn_prefill_q8k4v(cache, to_dev(w.q, w.dtype), to_dev(w.seq_lens), int(w.seq_lens.max()),
                                to_dev(w.page_table), w.softmax_scale, cfg=c)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _check(w, cache, oc, cfg, label):
    want = attention.verify(oc, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
    err = normalized_err(w, _prefill(w, cache, cfg), want)
    print(f"[prefill] {label} cfg {cfg}: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (label, cfg, err)


@pytest.mark.parametrize("hq,hkv,D,dt,n_new,lens", [
    (32, 8, 128, "bf16", 64, [700, 150]),
    (32, 4, 128, "bf16", 200, [2000]),
    (8, 8, 64, "f32", 37, [40, 500, 37]),
    (16, 2, 128, "bf16", 129, [900, 300]),
], ids=str)
def test_chunk_parity(hq, hkv, D, dt, n_new, lens):
    from tests.gpu_util import upload_cache
    w = workloads.build("prefill", seed=90 + n_new, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=dt,
                        seq_lens=[L + n_new for L in lens] if lens[0] != n_new else lens, n_draft=n_new,
                        outliers=True)
    cache, oc = upload_cache(w), oracle_cache(w)
    for cfg in (None, dict(variant=5, waves_per_wg=4), dict(variant=5, waves_per_wg=2, stages=3)):
        _check(w, cache, oc, cfg, f"Hq {hq} Hkv {hkv} D {D} n_new {n_new}")


def test_longest_chunk():
    from tests.gpu_util import upload_cache
    w = workloads.build("prefill_max", seed=95, num_q_heads=8, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1024 + 100], n_draft=1024, outliers=True)
    _check(w, upload_cache(w), oracle_cache(w), None, "n_new 1024")


def test_chunk_on_an_affine_cache():
    from tests.gpu_util import upload_cache
    w = workloads.build("prefill_aff", seed=96, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1500 + 100], n_draft=100, outliers=True)
    _check(w, upload_cache(w, codec="affine"), oracle_cache(w, codec_name="affine"), None, "affine n_new 100")
