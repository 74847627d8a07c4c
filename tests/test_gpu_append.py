"""GPU parity of kv_quant_append: codes and scales bit-exact with the oracle
on the named workloads, ragged multi-sequence batches with odd start slots,
and hand-built edge rows (zeros, ties, subnormal / underflowing / saturating
scales)."""

import numpy as np
import pytest

import workloads
from tests.util import oracle_cache

pytestmark = pytest.mark.gpu


def _assert_same(w, got, ref):
    assert np.array_equal(got["k_codes"], ref.k_codes), "key codes differ"
    assert np.array_equal(got["k_scales"], ref.k_scales), "key scales differ"
    assert np.array_equal(got["v_scales"], ref.v_scales), "value scales differ"
    assert np.array_equal(got["v_codes"], ref.v_codes), "value codes differ"


def _resplit(w, rng, pieces=3):
    """Split every append batch into `pieces` consecutive batches with random
    (often odd) cut points, so that appends start on odd slots and byte pairs
    are completed by a later call."""
    out = []
    for a in w.appends:
        B = len(a.start_pos)
        n = np.diff(a.cu_new)
        cuts = [np.sort(rng.integers(0, n[b] + 1, size=pieces - 1)) for b in range(B)]
        bounds = [np.concatenate([[0], c, [n[b]]]) for b, c in enumerate(cuts)]
        for p in range(pieces):
            rows, cnt = [], []
            for b in range(B):
                lo, hi = bounds[b][p], bounds[b][p + 1]
                rows.append(np.arange(a.cu_new[b] + lo, a.cu_new[b] + hi))
                cnt.append(hi - lo)
            rows = np.concatenate(rows).astype(np.int64)
            out.append(workloads.AppendBatch(
                k=a.k[rows], v=a.v[rows], cu_new=np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32),
                start_pos=(a.start_pos + np.array([bounds[b][p] for b in range(B)])).astype(np.int32),
                page_table=a.page_table))
    w.appends = out
    return w


@pytest.mark.parametrize("name", ["tiny_decode_256", "gqa_decode_4096"])
def test_named_workloads_bit_exact(name):
    from tests.gpu_util import cache_to_host, upload_cache
    w = workloads.NAMED[name]()
    print(f"[append] {name}", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32"), (128, "f32"), (64, "bf16")])
def test_ragged_batches_odd_starts(D, dtype):
    from tests.gpu_util import cache_to_host, upload_cache
    rng = np.random.default_rng(D + len(dtype))
    w = workloads.build("ragged", seed=31, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                        seq_lens=[1, 15, 16, 17, 33, 250, 0, 61], outliers=True, spare_pages=3)
    w = _resplit(w, rng)
    print(f"[append] ragged D={D} {dtype}", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32")])
def test_bulk_calls_mixed_chunks(D, dtype):
    """Calls of 256 tokens or more take the page-block kernel: one ragged call
    (sequences of 0..250 tokens from position 0: chunks that fill one page of
    one sequence and chunks that straddle sequences or pages), then longer
    sequences appended in two calls cut at random positions (odd starts)."""
    from tests.gpu_util import cache_to_host, upload_cache
    w = workloads.build("bulk_ragged", seed=41, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                        seq_lens=[1, 15, 16, 17, 33, 250, 0, 61], outliers=True)
    assert sum(len(a.k) for a in w.appends) >= 256
    print(f"[append] bulk ragged one call D={D} {dtype}", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))
    rng = np.random.default_rng(D)
    w = workloads.build("bulk_cut", seed=42, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                        seq_lens=[700, 333], outliers=True, spare_pages=2)
    w = _resplit(w, rng, pieces=2)
    print(f"[append] bulk two calls D={D} {dtype}: {[len(a.k) for a in w.appends]}", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))


def _edge_rows(D):
    rows = []
    z = np.zeros(D, np.float32)
    rows.append(z.copy())                                            # zero row
    r = z.copy(); r[:10] = [127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5, -126.5, 7]; rows.append(r)  # ties
    r = z.copy(); r[0] = 127 * 2.0 ** -20; r[1] = -6 * 2.0 ** -20; r[40] = 2 * 2.0 ** -20; rows.append(r)  # subnormal
    r = z.copy(); r[0] = 1e-9; r[3] = -5e-10; rows.append(r)                      # underflow
    r = z.copy(); r[0] = 1e7; r[1] = -65504; r[2] = 32752; r[33] = -3e6; rows.append(r)  # saturation
    rng = np.random.default_rng(4)
    for mag in (1e-6, 1e-3, 1.0, 1e3, 1e5):
        rows.append((rng.standard_normal(D) * mag).astype(np.float32))
    r = rng.standard_normal(D).astype(np.float32)                     # per-group ties for values
    for g in range(D // 32):
        r[32 * g] = 7.0 * 2 ** -g
        r[32 * g + 1: 32 * g + 8] = np.array([0.5, 1.5, 2.5, -3.5, 6.5, -6.5, 3.5]) * 2 ** -g
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("D", [64, 128])
def test_edge_rows_bit_exact(D):
    from tests.gpu_util import cache_to_host, upload_cache
    rows = _edge_rows(D)
    n = rows.shape[0]
    k = np.stack([rows, rows[::-1]], axis=1)            # [n][2][D]
    v = np.stack([rows[::-1], rows], axis=1)
    w = workloads.build("edge", seed=1, num_q_heads=2, num_kv_heads=2, head_dim=D, dtype="f32",
                        seq_lens=[n], permute_pages=True)
    w.appends = [workloads.AppendBatch(k=k.astype(np.float32), v=v.astype(np.float32),
                                       cu_new=np.array([0, n], np.int32), start_pos=np.array([0], np.int32),
                                       page_table=w.page_table)]
    print(f"[append] edge rows D={D}", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))


@pytest.mark.slow
def test_full_64k_cache_bit_exact():
    from tests.gpu_util import cache_to_host, upload_cache
    w = workloads.gqa_decode_64k()
    print("[append] gqa_decode_65536 full cache", flush=True)
    _assert_same(w, cache_to_host(upload_cache(w)), oracle_cache(w))
