"""Seeded synthetic workloads shared by the tests, the bench and the oracle.

This module only draws random inputs and lays out page tables: it holds none
of the method's arithmetic (no quantization, no attention).  Both the CPU
oracle and the HIP path consume exactly the arrays built here.

Recipe (numpy ``default_rng(seed)``; draw order fixed: queries, keys,
values, key outlier channels, value outlier channels, page permutation; the
multi-session suffix lengths come from ``default_rng(seed + 1000)``, those of
the tuner's session references from ``default_rng(seed + 3000)``):

* queries, keys and values are standard normal, drawn in float32;
* "outlier channels": ``round(0.01 * Hkv * D)`` (kv head, dim) channels are
  drawn without replacement, separately for keys and for values, and are
  multiplied by 8 in float32 for every token;
* bf16 workloads round the float32 draws to bfloat16 (nearest, ties to even)
  by bit arithmetic and hand the bit patterns over;
* physical page ids are a seeded permutation of the pool, so logical order
  and physical order differ; in the multi-session workload every session maps
  the same shared prefix pages first, then private suffix pages;
* optional query dynamic range (from its own stream, ``default_rng(seed +
  2000)``, so the draws above are unchanged): ``q_outlier`` multiplies
  ``round(0.01 * Hq * D)`` (query head, dim) channels, drawn without
  replacement, by that factor in every query row; ``q_decades`` multiplies
  every query element by 10 ** U(-q_decades / 2, q_decades / 2).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE_SIZE = 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the uint16 bit
    patterns.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@dataclass
class AppendBatch:
    """One call of quantize-and-append: rows cu_new[b]:cu_new[b+1] of k/v go to
    logical positions start_pos[b]... of sequence b (page table row b)."""
    k: np.ndarray            # [N][Hkv][D]  float32 or bf16 bits
    v: np.ndarray
    cu_new: np.ndarray       # [B+1] int32
    start_pos: np.ndarray    # [B] int32
    page_table: np.ndarray   # [B][max_pages] int32


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                       # "f32" or "bf16" (queries, keys, values)
    num_pages: int                   # physical pool size
    page_table: np.ndarray           # [B][max_pages] int32
    seq_lens: np.ndarray             # [B] int32, cached tokens attended
    q: np.ndarray                    # [B][Hq][D] or [B][W][Hq][D]
    n_draft: int                     # 0 = decode
    softmax_scale: float
    appends: List[AppendBatch] = field(default_factory=list)
    sigma_k: Optional[np.ndarray] = None   # [Hkv][D] generator std per channel
    sigma_v: Optional[np.ndarray] = None
    shared_prefix: int = 0

    @property
    def n_seqs(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def unique_tokens(self) -> int:
        """Distinct cached tokens (a shared prefix counted once)."""
        return int(np.sum(self.seq_lens) - self.shared_prefix * (self.n_seqs - 1)) \
            if self.shared_prefix else int(np.sum(self.seq_lens))


def _outlier_mask(rng, hkv, d):
    n = int(round(0.01 * hkv * d))
    idx = rng.choice(hkv * d, size=n, replace=False)
    m = np.ones(hkv * d, np.float32)
    m[idx] = 8.0
    return m.reshape(hkv, d)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def build(name: str, *, seed: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
          dtype: str, seq_lens, n_draft: int = 0, outliers: bool = False,
          shared_prefix: int = 0, permute_pages: bool = True, spare_pages: int = 0,
          value_scale: float = 1.0, q_outlier: float = 0.0, q_decades: float = 0.0) -> Workload:
    """Generic builder.  ``seq_lens`` counts cached tokens per sequence
    (drafts included for verify).  With ``shared_prefix`` > 0 (a multiple of
    16) every sequence maps the same prefix pages; each sequence's own tokens
    after the prefix are drawn per sequence."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int64)
    B = len(seq_lens)
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if shared_prefix % PAGE_SIZE:
        raise ValueError("shared prefix must be page aligned")
    if np.any(seq_lens < shared_prefix):
        raise ValueError("every sequence holds the shared prefix")
    if n_draft and np.any(seq_lens < n_draft):
        raise ValueError("verify sequences must hold their drafts")

    # -- draws, fixed order --------------------------------------------------
    qshape = (B, n_draft, Hq, D) if n_draft else (B, Hq, D)
    q = rng.standard_normal(qshape, dtype=np.float32)
    private = seq_lens - shared_prefix
    n_tok = shared_prefix + int(np.sum(private))
    k = rng.standard_normal((n_tok, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((n_tok, Hkv, D), dtype=np.float32) * np.float32(value_scale)
    if outliers:
        mk = _outlier_mask(rng, Hkv, D)
        mv = _outlier_mask(rng, Hkv, D)
        k *= mk[None]
        v *= mv[None]
    else:
        mk = np.ones((Hkv, D), np.float32)
        mv = np.ones((Hkv, D), np.float32)

    # -- pages ---------------------------------------------------------------
    pre_pages = shared_prefix // PAGE_SIZE
    per_seq_pages = [(int(L) - shared_prefix + PAGE_SIZE - 1) // PAGE_SIZE for L in seq_lens]
    num_pages = pre_pages + sum(per_seq_pages) + spare_pages
    max_pages = max(1, max(pre_pages + p for p in per_seq_pages))
    perm = rng.permutation(num_pages) if permute_pages else np.arange(num_pages)
    perm = perm.astype(np.int32)
    page_table = np.zeros((B, max_pages), np.int32)
    nxt = pre_pages
    for b in range(B):
        page_table[b, :pre_pages] = perm[:pre_pages]
        n = per_seq_pages[b]
        page_table[b, pre_pages:pre_pages + n] = perm[nxt:nxt + n]
        nxt += n

    # -- query dynamic range (own stream) ------------------------------------
    if q_outlier or q_decades:
        qrng = np.random.default_rng(seed + 2000)
        if q_outlier:
            n = int(round(0.01 * Hq * D))
            idx = qrng.choice(Hq * D, size=n, replace=False)
            m = np.ones(Hq * D, np.float32)
            m[idx] = np.float32(q_outlier)
            q *= m.reshape(Hq, D)
        if q_decades:
            q *= (10.0 ** qrng.uniform(-q_decades / 2, q_decades / 2, size=q.shape)).astype(np.float32)

    # -- append batches ------------------------------------------------------
    appends = []
    if shared_prefix:
        appends.append(AppendBatch(
            k=_encode(k[:shared_prefix], dtype), v=_encode(v[:shared_prefix], dtype),
            cu_new=np.array([0, shared_prefix], np.int32),
            start_pos=np.array([0], np.int32),
            page_table=page_table[:1].copy()))
    # private tokens: for verify the last n_draft of each sequence go in a
    # second batch (the drafts are appended right before they are verified)
    tail = n_draft
    body = private - tail
    offs = shared_prefix + np.concatenate([[0], np.cumsum(private)])
    rows_body = np.concatenate([np.arange(offs[b], offs[b] + body[b]) for b in range(B)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(body)]).astype(np.int32)
    if rows_body.size:
        appends.append(AppendBatch(
            k=_encode(k[rows_body], dtype), v=_encode(v[rows_body], dtype), cu_new=cu,
            start_pos=np.full(B, shared_prefix, np.int32), page_table=page_table))
    if tail:
        rows_tail = np.concatenate([np.arange(offs[b] + body[b], offs[b + 1]) for b in range(B)]).astype(np.int64)
        appends.append(AppendBatch(
            k=_encode(k[rows_tail], dtype), v=_encode(v[rows_tail], dtype),
            cu_new=(np.arange(B + 1) * tail).astype(np.int32),
            start_pos=(seq_lens - tail).astype(np.int32), page_table=page_table))

    return Workload(
        name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
        num_pages=num_pages, page_table=page_table, seq_lens=seq_lens.astype(np.int32),
        q=_encode(q, dtype), n_draft=n_draft,
        softmax_scale=float(np.float32(1.0 / np.sqrt(D))), appends=appends,
        sigma_k=mk, sigma_v=mv * np.float32(value_scale), shared_prefix=shared_prefix)


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def tiny_decode(seed: int = 0) -> Workload:
    """1 sequence, 2 query heads over 1 kv head, D 64, 256 tokens, fp32."""
    return build("tiny_decode_256", seed=seed, num_q_heads=2, num_kv_heads=1, head_dim=64,
                 dtype="f32", seq_lens=[256], permute_pages=False)


def gqa_decode(context: int, seed: int) -> Workload:
    """Batch 1, 32 query / 8 kv heads, D 128, bf16, 1 % outlier channels x8."""
    return build(f"gqa_decode_{context}", seed=seed, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, dtype="bf16", seq_lens=[context], outliers=True)


def gqa_decode_4k(seed: int = 1) -> Workload:
    return gqa_decode(4096, seed)


def gqa_decode_64k(seed: int = 2) -> Workload:
    return gqa_decode(65536, seed)


def verify_64k(seed: int = 3, context: int = 65536, n_draft: int = 8) -> Workload:
    """65536 cached tokens plus 8 drafts (appended first), causal among them."""
    return build(f"verify_{context}_w{n_draft}", seed=seed, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, dtype="bf16", seq_lens=[context + n_draft], n_draft=n_draft,
                 outliers=True)


def multi_session(seed: int = 4, sessions: int = 16, prefix: int = 32768,
                  max_suffix: int = 32768) -> Workload:
    """16 sessions, 32 query / 4 kv heads, one shared 32768-token prefix and
    a private suffix of uniform-random 0..32768 tokens each."""
    rng = np.random.default_rng(seed + 1000)
    suffix = rng.integers(0, max_suffix + 1, size=sessions)
    return build(f"multi_session_{sessions}x{prefix}", seed=seed, num_q_heads=32, num_kv_heads=4,
                 head_dim=128, dtype="bf16", seq_lens=prefix + suffix, outliers=True,
                 shared_prefix=prefix)


def tune_reference(context: int, n_draft: int = 8, seed: int = 11) -> Workload:
    """Caller inputs of the tuner's oracle gate at one context: one sequence
    of ``context`` cached tokens plus ``n_draft`` drafts (32 query / 8 kv
    heads, D 128, bf16, 1 % outlier channels x8).  The decode term attends
    the first ``context`` tokens with draft 0's query, the verify term all of
    them with every draft."""
    return build(f"tune_ref_{context}_w{n_draft}", seed=seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 dtype="bf16", seq_lens=[context + n_draft], n_draft=n_draft, outliers=True)


def multi_session_part(part: str, seed: int = 4, sessions: int = 16, prefix: int = 32768,
                       max_suffix: int = 32768) -> Workload:
    """One of the two passes of the 16-session workload on its own: "prefix"
    -- every session the shared prefix and one token of its own (the
    cascade's suffix pass is a single page per session) -- or "suffixes" --
    the sessions' private suffixes (same lengths as the full workload) as
    plain sequences without the prefix."""
    rng = np.random.default_rng(seed + 1000)
    suffix = rng.integers(0, max_suffix + 1, size=sessions)
    if part == "prefix":
        return build(f"multi_session_{sessions}x{prefix}_prefix", seed=seed, num_q_heads=32, num_kv_heads=4,
                     head_dim=128, dtype="bf16", seq_lens=np.full(sessions, prefix + 1), outliers=True,
                     shared_prefix=prefix)
    return build(f"multi_session_{sessions}_suffixes", seed=seed, num_q_heads=32, num_kv_heads=4, head_dim=128,
                 dtype="bf16", seq_lens=suffix, outliers=True)


def tune_sessions_reference(context: int, sessions: int = 16, seed: int = 13) -> Workload:
    """Caller inputs of the tuner's multi-session oracle terms at one context:
    ``sessions`` sessions (32 query / 4 kv heads, D 128, bf16, 1 % outlier
    channels x8) over one ``context / 2`` token shared prefix, each with a
    private suffix of uniform-random 1..context/2 tokens (the length mix of
    the 16-session workload, at ``context`` 65536)."""
    half = context // 2
    rng = np.random.default_rng(seed + 3000)
    suffix = rng.integers(1, half + 1, size=sessions)
    return build(f"tune_ref_sessions_{sessions}x{half}", seed=seed, num_q_heads=32, num_kv_heads=4, head_dim=128,
                 dtype="bf16", seq_lens=half + suffix, outliers=True, shared_prefix=half)


NAMED = {
    "tiny_decode_256": tiny_decode,
    "gqa_decode_4096": gqa_decode_4k,
    "gqa_decode_65536": gqa_decode_64k,
    "verify_65536_w8": verify_64k,
    "multi_session_16x32768": multi_session,
    # longer contexts of the same shapes (timed on request, not in every run)
    "gqa_decode_131072": lambda: gqa_decode(131072, 5),
    "gqa_decode_200000": lambda: gqa_decode(200000, 6),
    "verify_131072_w8": lambda: verify_64k(7, 131072, 8),
    "verify_200000_w8": lambda: verify_64k(8, 200000, 8),
    # a uniform batch: 16 sequences of 4096 tokens (as many cache bytes as the 64K decode)
    "batch_decode_16x4096": lambda: build("batch_decode_16x4096", seed=9, num_q_heads=32, num_kv_heads=8,
                                          head_dim=128, dtype="bf16", seq_lens=[4096] * 16, outliers=True),
    # the 16-session workload's two passes on their own
    "multi_session_16x32768_prefix": lambda: multi_session_part("prefix"),
    "multi_session_16_suffixes": lambda: multi_session_part("suffixes"),
}
