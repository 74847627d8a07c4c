"""Softmax attention over the dequantized paged cache, fp64, CPU reference.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

The method does not approximate attention: given the quantized cache, decode
attention is exact softmax attention over the dequantized keys and values
(the only approximation is the codec, reproduced bit-exactly in
``oracle.codec``).  So this module is the textbook definition written out:

    score_t = c * sum_d q_d * khat_{t,d}        (c: the fp32 softmax scale, widened)
    w_t     = exp(score_t - max_u score_u)
    o_d     = sum_t w_t * vhat_{t,d} / sum_t w_t

Speculative verify (blog.123qwe.co.kr/?p=3927, section 5: checking several
draft tokens in one pass, at the cost of one decode step because decode is
bound by memory traffic) attends the same cache with W draft queries.
Reading for the causal rule among the drafts: the drafts' own keys/values are
appended first, so a sequence holding L cached tokens verifies drafts at
positions L-W .. L-1, and draft j (0-based) sees positions 0 .. L-W+j.

GQA mapping (the workloads use 32 query heads over 8 or 4 kv heads): query
head h reads kv head h // (Hq / Hkv), i.e. contiguous groups.
"""

from __future__ import annotations

import numpy as np

from .codec import PAGE_SIZE, PagedCache, as_f32


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One query row ``q [D]`` over ``k, v [T][D]`` (all fp64) -> ``[D]``."""
    s = scale * (k @ q)
    m = np.max(s)
    w = np.exp(s - m)
    return (w @ v) / np.sum(w)


def sequence_kv(cache: PagedCache, page_table_row: np.ndarray, length: int, h: int):
    """fp64 K-hat, V-hat ``[length][D]`` of kv head h, gathered through the
    page table in logical order."""
    pos = np.arange(length, dtype=np.int64)
    pages = np.asarray(page_table_row, np.int64)[pos // PAGE_SIZE]
    return cache.dequant_tokens(pages, pos % PAGE_SIZE, h)


def _scale64(softmax_scale: float) -> float:
    return float(np.float32(softmax_scale))


def decode(cache: PagedCache, q: np.ndarray, q_dtype: str, page_table: np.ndarray,
           seq_lens: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Decode attention, one query token per sequence.

    ``q`` is ``[B][Hq][D]`` (float32 values or bf16 bit patterns); sequence b
    attends its first ``seq_lens[b]`` cached tokens.  Returns fp64
    ``[B][Hq][D]``; a sequence of length 0 yields zeros."""
    qf = as_f32(q, q_dtype).astype(np.float64)
    B, Hq, D = qf.shape
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    c = _scale64(softmax_scale)
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for kvh in range(Hkv):
            kh, vh = sequence_kv(cache, page_table[b], L, kvh)
            for g in range(G):
                h = kvh * G + g
                out[b, h] = softmax_attention(qf[b, h], kh, vh, c)
    return out


def verify(cache: PagedCache, q: np.ndarray, q_dtype: str, page_table: np.ndarray,
           seq_lens: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Verify attention for W draft queries per sequence.

    ``q`` is ``[B][W][Hq][D]``; ``seq_lens[b]`` counts the cached tokens
    including the W drafts.  Draft j attends positions ``0 .. L-W+j``.
    Returns fp64 ``[B][W][Hq][D]``."""
    qf = as_f32(q, q_dtype).astype(np.float64)
    B, W, Hq, D = qf.shape
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    c = _scale64(softmax_scale)
    out = np.zeros((B, W, Hq, D), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < W:
            raise ValueError("a verify sequence must hold at least its W drafts")
        for kvh in range(Hkv):
            kh, vh = sequence_kv(cache, page_table[b], L, kvh)
            for j in range(W):
                vis = L - W + j + 1
                for g in range(G):
                    h = kvh * G + g
                    out[b, j, h] = softmax_attention(qf[b, j, h], kh[:vis], vh[:vis], c)
    return out
