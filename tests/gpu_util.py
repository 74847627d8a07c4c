"""Device-side helpers for the GPU tests: upload a workload through the
library's own append entry point and read results back."""

import numpy as np
import torch

import decode_attention_quantized_kv_amd as q8


def to_dev(a: np.ndarray, dtype: str = None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def upload_cache(w, extra_pages: int = 0, codec: str = "symmetric") -> q8.PagedKVCache:
    cache = q8.PagedKVCache(w.num_pages + extra_pages, w.num_kv_heads, w.head_dim, codec=codec)
    for a in w.appends:
        q8.kv_quant_append(cache, to_dev(a.k, w.dtype), to_dev(a.v, w.dtype), to_dev(a.cu_new),
                           to_dev(a.start_pos), to_dev(a.page_table))
    torch.cuda.synchronize()
    return cache


def cache_to_host(cache: q8.PagedKVCache) -> dict:
    d = {
        "k_codes": cache.k_codes.cpu().numpy(),
        "k_scales": cache.k_scales.cpu().numpy().view(np.uint16),
        "v_codes": cache.v_codes.cpu().numpy(),
        "v_scales": cache.v_scales.cpu().numpy().view(np.uint16),
    }
    if cache.codec == "affine":
        d["k_zeros"] = cache.k_zeros.cpu().numpy()
        d["v_zeros"] = cache.v_zeros.cpu().numpy()
    return d


def run_attention(w, cache, cfg=None, q=None, seq_lens=None, max_seq_len=None):
    q = to_dev(w.q if q is None else q, w.dtype)
    lens = to_dev(w.seq_lens if seq_lens is None else seq_lens)
    pt = to_dev(w.page_table)
    msl = int(max(w.seq_lens)) if max_seq_len is None else max_seq_len
    if q.dim() == 4:
        out = q8.attn_verify_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=cfg)
    else:
        out = q8.attn_decode_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_prefix(w, cache, n_prefix_pages, cfg=None, max_seq_len=None):
    """attn_decode_prefix_q8k4v on a decode workload whose sequences share
    their first n_prefix_pages pages."""
    q = to_dev(w.q, w.dtype)
    lens = to_dev(w.seq_lens)
    pt = to_dev(w.page_table)
    msl = int(max(w.seq_lens)) if max_seq_len is None else max_seq_len
    out = q8.attn_decode_prefix_q8k4v(cache, q, lens, msl, pt, n_prefix_pages, w.softmax_scale, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)
