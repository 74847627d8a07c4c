"""HIP-graph capture of the hot-path calls: every replay of a captured
decode (separate and fused split merge), verify, shared-prefix cascade and
append reproduces the eager result bit for bit, with eager work and
synchronisations between the replays (the calls record no memset and leave
the fused-merge counters at zero, so a graph can be replayed as is)."""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _replays_match(fn, out, n=4):
    import torch
    fn()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm the stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"
        fn()                                   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [None, dict(fused_combine=1), dict(variant=5)], ids=str)
def test_decode_graph_replays(cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.build("graph_dec", seed=41, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[5000, 1200], outliers=True)
    cache = upload_cache(w)
    q, lens, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
    c = None if cfg is None else q8.make_config(**cfg)
    msl = int(w.seq_lens.max())
    ws = q8._workspace(q8.workspace_bytes(w.n_seqs, 32, 8, 128, msl, 0, c), q.device)
    out = q8.attn_decode_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=c, workspace=ws)
    _replays_match(lambda: q8.attn_decode_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, out=out, cfg=c,
                                                workspace=ws), out)


def test_verify_graph_replays():
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.build("graph_ver", seed=42, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[4100], n_draft=8, outliers=True)
    cache = upload_cache(w)
    q, lens, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
    msl = int(w.seq_lens.max())
    ws = q8._workspace(q8.workspace_bytes(1, 32, 8, 128, msl, 8), q.device)
    out = q8.attn_verify_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, workspace=ws)
    _replays_match(lambda: q8.attn_verify_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, out=out, workspace=ws),
                   out)


def test_cascade_graph_replays():
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.multi_session(seed=43, sessions=6, prefix=512, max_suffix=900)
    cache = upload_cache(w)
    q, lens, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
    msl, npre = int(w.seq_lens.max()), w.shared_prefix // 16
    ws = q8._workspace(q8.prefix_workspace_bytes(w.n_seqs, w.num_q_heads, w.num_kv_heads, 128, msl, npre), q.device)
    out = q8.attn_decode_prefix_q8k4v(cache, q, lens, msl, pt, npre, w.softmax_scale, workspace=ws)
    _replays_match(lambda: q8.attn_decode_prefix_q8k4v(cache, q, lens, msl, pt, npre, w.softmax_scale, out=out,
                                                       workspace=ws), out)


def test_append_graph_replays():
    """The appends of a whole workload captured in one graph rebuild the
    eagerly built cache bit for bit on every replay."""
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.build("graph_app", seed=44, num_q_heads=8, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[300, 77], n_draft=3, outliers=True)
    want = upload_cache(w)
    cache = q8.PagedKVCache(w.num_pages, w.num_kv_heads, w.head_dim)
    batches = [(to_dev(a.k, "bf16"), to_dev(a.v, "bf16"), to_dev(a.cu_new), to_dev(a.start_pos),
                to_dev(a.page_table)) for a in w.appends]
    assert len(batches) >= 2
    pools = lambda c: (c.k_codes, c.k_scales, c.v_codes, c.v_scales)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for (k, v, cu, sp, pt) in batches:
            q8.kv_quant_append(cache, k, v, cu, sp, pt)
    for i in range(3):
        for t in pools(cache):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t, ref in zip(pools(cache), pools(want)):
            assert torch.equal(t, ref), f"replay {i}"
