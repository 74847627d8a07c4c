"""The attention kernels round each query row to a fixed-point number before
the int8 MFMA on the stored key codes: Q = rne(q * 2^(b - e)) with
2^(e-1) <= max|q_row| < 2^e.  This CPU check evaluates that rounding rule
with the oracle's own attention (exact query vs rounded query, same quantized
cache) on queries with a wide dynamic range -- 1 % of the channels x64 and
x1024 (bf16), and fp32 queries spread over six decades -- and shows

* with the kernels' 23-bit form (b = 22) the output stays within the 2e-3
  sigma tolerance and within the derived bound
  |dout| <= (exp(2 max|ds|) - 1) max|v|,  |ds| <= c 2^(e - 23) ||k||_1;
* the two-digit 15-bit form (b = 14) leaves the tolerance on these inputs,
  which is why the kernels carry a third int8 digit.

It tests a rounding rule, not the kernels (their GPU parity on the same kind
of queries is tests/test_gpu_query_range.py); the attention is the oracle's.
"""

import numpy as np
import pytest

import workloads
from oracle import attention, codec
from tests.util import ATOL_SIGMA, oracle_cache, sigma_q_heads


def _rounded(q: np.ndarray, bits: int) -> np.ndarray:
    mx = float(np.max(np.abs(q)))
    e = np.frexp(mx)[1] if mx > 0 else 0          # 2^(e-1) <= mx < 2^e
    return np.rint(q * 2.0 ** (bits - e)) * 2.0 ** (e - bits), e


def _workload(mult: float, dtype: str, wide: bool, seed: int = 5, ctx: int = 4096):
    w = workloads.build("q_range", seed=seed, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=dtype,
                        seq_lens=[ctx], outliers=True,
                        q_outlier=0.0 if wide else mult, q_decades=6.0 if wide else 0.0)
    return w


def _decode_rounded(w, cache, bits):
    """Per q head: the oracle's softmax attention with the rounded query row,
    and the bound on the output change that rounding can cause."""
    qf = codec.as_f32(w.q, w.dtype).astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    c = float(np.float32(w.softmax_scale))
    L = int(w.seq_lens[0])
    out = np.zeros_like(qf)
    bound = np.zeros(qf.shape[:2])
    for kvh in range(w.num_kv_heads):
        kh, vh = attention.sequence_kv(cache, w.page_table[0], L, kvh)
        k1 = float(np.max(np.sum(np.abs(kh), axis=1)))
        vmax = float(np.max(np.abs(vh)))
        for g in range(G):
            h = kvh * G + g
            Q, e = _rounded(qf[0, h], bits)
            out[0, h] = attention.softmax_attention(Q, kh, vh, c)
            ds = c * 2.0 ** (e - bits - 1) * k1
            bound[0, h] = np.expm1(2.0 * ds) * vmax
    return out, bound


CASES = [(64.0, "bf16", False), (1024.0, "bf16", False), (1.0, "f32", True)]


@pytest.mark.parametrize("mult,dtype,wide", CASES, ids=["bf16_x64", "bf16_x1024", "f32_six_decades"])
def test_kernel_rounding_stays_in_tolerance_and_bound(mult, dtype, wide):
    w = _workload(mult, dtype, wide)
    cache = oracle_cache(w)
    want = attention.decode(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
    got, bound = _decode_rounded(w, cache, 22)
    err = np.abs(got - want)
    assert np.max(err / sigma_q_heads(w)) <= ATOL_SIGMA
    assert np.all(err <= bound[..., None] * (1 + 1e-9) + 1e-15)


def test_two_digit_rounding_leaves_the_tolerance():
    worst = 0.0
    for mult, dtype, wide in CASES:
        w = _workload(mult, dtype, wide)
        cache = oracle_cache(w)
        want = attention.decode(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
        got, _ = _decode_rounded(w, cache, 14)
        worst = max(worst, float(np.max(np.abs(got - want) / sigma_q_heads(w))))
    assert worst > ATOL_SIGMA
