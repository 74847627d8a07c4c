"""GPU parity for concurrent sessions sharing a prefix (blog.123qwe.co.kr/?p=3927,
section 5: sessions that share a prompt prefix read the same cached pages):
ragged multi-session decode against the fp64 oracle on every kernel, shared
prefix pages equal private copies bit for bit, and the full 16-session
workload (32768-token shared prefix, ragged suffixes up to 32768)."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[multi] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (label, err)


@pytest.mark.parametrize("cfg", [None, dict(variant=5), dict(variant=5, waves_per_wg=2, stages=3),
                                 dict(fused_combine=1), dict(variant=4, stages=2, waves_per_wg=2)], ids=str)
def test_ragged_sessions_with_shared_prefix(cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.multi_session(seed=12, sessions=6, prefix=256, max_suffix=700)
    assert w.shared_prefix == 256 and len(set(w.seq_lens.tolist())) > 1
    c = None if cfg is None else q8.make_config(**cfg)
    _check(w, run_attention(w, upload_cache(w), cfg=c), oracle_out(w), f"6 sessions cfg {cfg}")


def test_shared_prefix_equals_private_copies():
    """The same sessions with the prefix pages copied per session give the
    same output bit for bit (page ids are pure indexing)."""
    import torch
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.multi_session(seed=13, sessions=5, prefix=320, max_suffix=400)
    pre = w.shared_prefix // 16
    extra = (w.n_seqs - 1) * pre
    cache = upload_cache(w, extra_pages=extra)
    shared = run_attention(w, cache)
    # copy the prefix pages of sessions 1.. to fresh physical pages
    pt = w.page_table.copy()
    fresh = w.num_pages
    for b in range(1, w.n_seqs):
        src = torch.from_numpy(pt[b, :pre].astype(np.int64)).cuda()
        dst = torch.arange(fresh, fresh + pre, device="cuda")
        for pool in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales):
            pool[dst] = pool[src]
        pt[b, :pre] = np.arange(fresh, fresh + pre, dtype=np.int32)
        fresh += pre
    torch.cuda.synchronize()
    w.page_table = pt
    private = run_attention(w, cache)
    assert np.array_equal(shared, private)


@pytest.mark.slow
def test_full_multi_session_16x32768():
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.multi_session()
    cache = upload_cache(w)
    _check(w, run_attention(w, cache), oracle_out(w), "multi_session_16x32768")
