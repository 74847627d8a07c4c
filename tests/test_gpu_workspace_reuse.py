"""GPU parity with one workspace shared by every plan.

A caller that serves decode and verify (blog.123qwe.co.kr/?p=3927, section
5) at several context lengths keeps one workspace, zeroes it once and passes
it to every call.  The in-launch split merge counts arrivals in the
workspace header; every plan's split records lie behind that header, and
every completed launch leaves the counters at zero.  Here one workspace,
zeroed once, serves in turn: the 64K verify with the separate combine, the
4K and 64K decodes with the in-launch merge, the shared-prefix cascade, the
4K decode again and the 64K verify with the in-launch merge -- each against
the fp64 oracle, and the header is zero again at the end."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WS_HEADER = 65536        # Q8K4V_WS_HEADER_BYTES


def test_one_workspace_for_every_plan():
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache

    ver = workloads.verify_64k()
    d4 = workloads.gqa_decode_4k()
    d64 = workloads.gqa_decode_64k()
    ms = workloads.multi_session(seed=27, sessions=6, prefix=4096, max_suffix=3000)
    fused, plain = q8.make_config(fused_combine=1), q8.make_config(fused_combine=0)
    need = max(q8.workspace_bytes(1, 32, 8, 128, int(ver.seq_lens.max()), 8, plain),
               q8.workspace_bytes(1, 32, 8, 128, int(ver.seq_lens.max()), 8, fused),
               q8.workspace_bytes(1, 32, 8, 128, 4096, 0, fused),
               q8.workspace_bytes(1, 32, 8, 128, 65536, 0, fused),
               q8.prefix_workspace_bytes(ms.n_seqs, 32, 4, 128, int(ms.seq_lens.max()), ms.shared_prefix // 16))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")       # zeroed once
    ws[WS_HEADER:].fill_(0xFF)                                    # records: NaN until written

    caches = {}

    def run(w, cfg, label):
        if w.name not in caches:
            caches[w.name] = (upload_cache(w), oracle_out(w))
        cache, want = caches[w.name]
        q, sl, pt = to_dev(w.q, w.dtype), to_dev(w.seq_lens), to_dev(w.page_table)
        msl = int(w.seq_lens.max())
        if w.n_draft:
            out = q8.attn_verify_q8k4v(cache, q, sl, msl, pt, w.softmax_scale, cfg=cfg, workspace=ws)
        elif w.shared_prefix:
            out = q8.attn_decode_prefix_q8k4v(cache, q, sl, msl, pt, w.shared_prefix // 16, w.softmax_scale,
                                              workspace=ws)
        else:
            out = q8.attn_decode_q8k4v(cache, q, sl, msl, pt, w.softmax_scale, cfg=cfg, workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = normalized_err(w, got, want)
        print(f"[workspace reuse] {label}: max |err|/sigma = {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)), label
        assert err <= ATOL_SIGMA, (label, err)

    run(ver, plain, "64K verify, separate combine")
    run(d4, fused, "4K decode, in-launch merge")
    run(d64, fused, "64K decode, in-launch merge")
    run(ms, None, "6-session cascade")
    run(d4, fused, "4K decode again, in-launch merge")
    run(ver, fused, "64K verify, in-launch merge")
    run(d64, plain, "64K decode, separate combine")
    run(d64, fused, "64K decode, in-launch merge again")
    assert int(ws[:WS_HEADER].count_nonzero()) == 0      # every counter back at zero
