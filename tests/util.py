"""Helpers shared by the tests: build the oracle's cache for a workload and
the tolerance check used for attention outputs."""

import numpy as np

from oracle import attention, codec

# Attention output tolerance: max over elements of |o_gpu - o_oracle| / sigma_d
# <= 2e-3, where sigma_d is the generator's standard deviation of value
# channel d (8 for outlier channels, else the value scale).
ATOL_SIGMA = 2e-3


def oracle_cache(w, extra_pages: int = 0, codec_name: str = "symmetric") -> codec.PagedCache:
    cache = codec.PagedCache(w.num_pages + extra_pages, w.num_kv_heads, w.head_dim, codec=codec_name)
    for a in w.appends:
        codec.append(cache, a.k, a.v, w.dtype, a.cu_new, a.start_pos, a.page_table)
    return cache


def oracle_out(w, cache=None):
    cache = cache if cache is not None else oracle_cache(w)
    if w.n_draft:
        return attention.verify(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
    return attention.decode(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)


def sigma_q_heads(w) -> np.ndarray:
    """[Hq][D] value-channel sigma seen by each query head."""
    G = w.num_q_heads // w.num_kv_heads
    return np.repeat(w.sigma_v.astype(np.float64), G, axis=0)


def normalized_err(w, got, want) -> float:
    sig = sigma_q_heads(w)
    return float(np.max(np.abs(np.asarray(got, np.float64) - want) / sig)) if want.size else 0.0
