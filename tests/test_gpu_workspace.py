"""GPU parity with a workspace that holds garbage.  The decode and verify
units (blog.123qwe.co.kr/?p=3927, section 5) run split-K here, with a
log-sum-exp merge of the split records.  Splits past a sequence's last page
never write their records, so the merge must mask them rather than read
them.  The workspace's records are filled with 0xFF bytes (every float a
NaN) before each call, its header (the in-launch merge's counters) zeroed
as the contract asks; ragged batches with empty, one-token and long
sequences leave many such records."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


WS_HEADER = 65536        # Q8K4V_WS_HEADER_BYTES: zero before first use (the contract)


def _nan_workspace(nbytes):
    """The header zeroed as the contract asks, every record byte 0xFF."""
    import torch
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    ws[:WS_HEADER].zero_()
    return ws


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[workspace] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert err <= ATOL_SIGMA, (label, err)


@pytest.mark.parametrize("n_draft", [0, 4])
@pytest.mark.parametrize("cfg", [None, dict(variant=5), dict(split_pages=4), dict(fused_combine=1)], ids=str)
def test_garbage_workspace_decode_and_verify(n_draft, cfg):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    lens = [3000 + n_draft, 17 + n_draft, n_draft, 900 + n_draft, 1 + n_draft, 4096 + n_draft]
    w = workloads.build("wsnan", seed=41 + n_draft, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                        seq_lens=lens, n_draft=n_draft, outliers=True)
    cache = upload_cache(w)
    c = None if cfg is None else q8.make_config(**cfg)
    B = w.n_seqs
    msl = int(max(w.seq_lens))
    q, sl, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
    ws = _nan_workspace(q8.workspace_bytes(B, 16, 4, 128, msl, n_draft, c))
    if n_draft:
        out = q8.attn_verify_q8k4v(cache, q, sl, msl, pt, w.softmax_scale, cfg=c, workspace=ws)
    else:
        out = q8.attn_decode_q8k4v(cache, q, sl, msl, pt, w.softmax_scale, cfg=c, workspace=ws)
    torch.cuda.synchronize()
    _check(w, out.cpu().numpy().astype(np.float64), oracle_out(w), f"n_draft {n_draft} cfg {cfg}")


def test_garbage_workspace_shared_prefix():
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.multi_session(seed=23, sessions=7, prefix=512, max_suffix=900)
    cache = upload_cache(w)
    B, Hq = w.n_seqs, w.q.shape[1]
    msl = int(max(w.seq_lens))
    npp = w.shared_prefix // 16
    ws = _nan_workspace(q8.prefix_workspace_bytes(B, Hq, cache.num_kv_heads, cache.head_dim, msl, npp))
    out = q8.attn_decode_prefix_q8k4v(cache, to_dev(w.q, w.dtype), to_dev(w.seq_lens), msl, to_dev(w.page_table),
                                      npp, w.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    _check(w, out.cpu().numpy().astype(np.float64), oracle_out(w), "shared prefix, 7 sessions")
