"""GPU parity of attn_decode_append_q8k4v (one decode step: append each
sequence's new token, then decode over the cache including it; the decode
unit over the k8v4 cache of blog.123qwe.co.kr/?p=3927, section 5): the cache
afterwards equals kv_quant_append's bit for bit, the output equals the
separate append + decode bit for bit and the fp64 oracle within tolerance --
on the fused plan and on the plans that fall back to two launches, with new
tokens on odd and even slots and on the first slot of a page."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


def _split_last(w):
    """The workload's appends without each sequence's last token, and that
    token's K and V rows [B][H][D]."""
    last = w.appends[-1]
    B = len(last.start_pos)
    n = np.diff(last.cu_new)
    assert np.all(n >= 1)
    keep = np.concatenate([np.arange(last.cu_new[b], last.cu_new[b + 1] - 1) for b in range(B)]).astype(np.int64)
    rows = (last.cu_new[1:] - 1).astype(np.int64)
    head = workloads.AppendBatch(k=last.k[keep], v=last.v[keep],
                                 cu_new=np.concatenate([[0], np.cumsum(n - 1)]).astype(np.int32),
                                 start_pos=last.start_pos, page_table=last.page_table)
    return w.appends[:-1] + [head], last.k[rows], last.v[rows]


def _run(w, cfg, codec="symmetric"):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import cache_to_host, to_dev, upload_cache
    full = upload_cache(w, codec=codec)                    # the append kernel, every token
    appends, k_last, v_last = _split_last(w)
    w_step = workloads.Workload(**{**w.__dict__, "appends": appends})
    cache = upload_cache(w_step, codec=codec)
    c = None if cfg is None else q8.make_config(**cfg)
    q, lens, pt = to_dev(w.q, w.dtype), to_dev(w.seq_lens), to_dev(w.page_table)
    msl = int(w.seq_lens.max())
    got = q8.attn_decode_append_q8k4v(cache, to_dev(k_last, w.dtype), to_dev(v_last, w.dtype), q, lens, msl, pt,
                                      w.softmax_scale, cfg=c)
    sep = q8.attn_decode_q8k4v(full, q, lens, msl, pt, w.softmax_scale, cfg=c)
    torch.cuda.synchronize()
    a, b = cache_to_host(cache), cache_to_host(full)
    for name in a:
        assert np.array_equal(a[name], b[name]), f"{name} differ from kv_quant_append's"
    return got.cpu().numpy().astype(np.float64), sep.cpu().numpy().astype(np.float64)


CFGS = [None, dict(fused_combine=1), dict(split_pages=4096), dict(variant=4, stages=3), dict(variant=4, waves_per_wg=8),
        dict(variant=5), dict(variant=5, waves_per_wg=8, fused_combine=1)]


@pytest.mark.parametrize("cfg", CFGS, ids=str)
def test_step_matches_append_then_decode(cfg):
    w = workloads.build("dec_app", seed=101, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1, 2, 16, 17, 32, 33, 500, 2049], outliers=True)
    got, sep = _run(w, cfg)
    assert np.array_equal(got, sep), cfg
    err = normalized_err(w, got, oracle_out(w))
    print(f"[decode_append] cfg {cfg}: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (cfg, err)


@pytest.mark.parametrize("hq,hkv,D,dt", [(8, 8, 64, "f32"), (32, 4, 128, "bf16"), (16, 8, 64, "bf16"),
                                         (16, 2, 128, "f32")], ids=str)
def test_groups_heads_dtypes(hq, hkv, D, dt):
    w = workloads.build("dec_app_g", seed=102 + hq + D, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=dt,
                        seq_lens=[3, 64, 65, 1000], outliers=True)
    got, sep = _run(w, None)
    assert np.array_equal(got, sep)
    assert normalized_err(w, got, oracle_out(w)) <= ATOL_SIGMA


@pytest.mark.parametrize("hq,hkv,D,dt,cfg", [(32, 8, 128, "bf16", None), (8, 8, 64, "f32", None),
                                             (32, 8, 128, "bf16", dict(variant=4, waves_per_wg=8))], ids=str)
def test_affine_cache(hq, hkv, D, dt, cfg):
    """Affine codec: the fused step writes the token's codes, scales and zero
    points as kv_quant_append does (bit for bit), and its output equals the
    separate append + decode and the oracle over the affine cache."""
    from tests.util import oracle_cache
    w = workloads.build("dec_app_aff", seed=140 + D, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype=dt,
                        seq_lens=[1, 2, 16, 17, 33, 700], outliers=True)
    got, sep = _run(w, cfg, codec="affine")
    assert np.array_equal(got, sep), cfg
    err = normalized_err(w, got, oracle_out(w, oracle_cache(w, codec_name="affine")))
    print(f"[decode_append] affine hq={hq} D={D} {dt} cfg {cfg}: {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, err


def test_graph_replays_rewrite_the_same_token():
    """Captured in a graph and replayed, the step rewrites the same codes and
    gives the same output every time."""
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.build("dec_app_graph", seed=103, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[3000, 77], outliers=True)
    cache = upload_cache(w)
    _, k_last, v_last = _split_last(w)
    kn, vn = to_dev(k_last, "bf16"), to_dev(v_last, "bf16")
    q, lens, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
    msl = int(w.seq_lens.max())
    ws = q8._workspace(q8.workspace_bytes(2, 32, 8, 128, msl, 0), q.device)
    out = q8.attn_decode_append_q8k4v(cache, kn, vn, q, lens, msl, pt, w.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    want = out.clone()
    pools = [t.clone() for t in cache.pools()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.attn_decode_append_q8k4v(cache, kn, vn, q, lens, msl, pt, w.softmax_scale, out=out, workspace=ws)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"
        for t, ref in zip(cache.pools(), pools):
            assert torch.equal(t, ref)
