"""GPU parity when the scores climb or fall along the sequence.  The kernels'
online softmax keeps a per-row reference that moves only when a score passes
it (and then lands a fixed headroom above the new maximum), so these inputs
drive every branch of it: scores that climb faster than the headroom on every
two-page tile (a rescale on each tile), scores that climb slowly (the
reference moves now and then), and scores that fall (the first tile sets it
for good), each with a knee after which the scores stay level so that many
tokens share the softmax mass.  Decode, verify and the shared-prefix cascade,
with splits long enough that each wave walks several tiles, against the fp64
oracle (blog.123qwe.co.kr/?p=3927, section 4: the attention the quantized
cache stands in for)."""

import numpy as np
import pytest

import workloads
from oracle import attention, codec
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache, oracle_out

LOG2E = 1.4426950408889634
# score slopes along the sequence, log2 units per token: 0.1 gains 3.2 per
# 32-token tile (more than the headroom), 0.004 gains 0.13, -0.05 falls
SLOPES = [0.1, 0.004, -0.05]


def _ramp(w, slope: float, knee: int, seed: int):
    """Give the queries and keys of each kv head a common unit direction u:
    queries become 0.2 q + u, keys gain a(pos) u with a chosen so that the
    score of the token at pos gains about slope * min(pos, knee) (log2
    units).  f32 workloads only (the arrays are edited in place)."""
    assert w.dtype == "f32"
    rng = np.random.default_rng(seed)
    Hkv, D = w.num_kv_heads, w.head_dim
    G = w.num_q_heads // Hkv
    u = rng.standard_normal((Hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    uq = np.repeat(u, G, axis=0).astype(np.float32)               # [Hq][D]
    w.q[...] = np.float32(0.2) * w.q + uq
    per = slope / (w.softmax_scale * LOG2E)
    for a in w.appends:
        for b in range(len(a.start_pos)):
            lo, hi = int(a.cu_new[b]), int(a.cu_new[b + 1])
            pos = int(a.start_pos[b]) + np.arange(hi - lo)
            amp = (per * np.minimum(pos, knee)).astype(np.float32)
            a.k[lo:hi] += amp[:, None, None] * u[None].astype(np.float32)
    return w


def _decode_workload(slope, seed):
    w = workloads.build(f"ramp_dec_{slope}", seed=seed, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="f32",
                        seq_lens=[2100, 700, 90])
    return _ramp(w, slope, knee=1200, seed=seed + 1)


def _verify_workload(slope, seed):
    w = workloads.build(f"ramp_ver_{slope}", seed=seed, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="f32",
                        seq_lens=[2100, 600], n_draft=8)
    return _ramp(w, slope, knee=1200, seed=seed + 1)


def _sessions_workload(slope, seed):
    w = workloads.build(f"ramp_sess_{slope}", seed=seed, num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="f32",
                        seq_lens=[1024 + 5, 1024 + 400, 1024 + 1100, 1024], shared_prefix=1024)
    return _ramp(w, slope, knee=1500, seed=seed + 1)


def test_fast_ramp_passes_the_headroom_on_every_tile():
    """CPU check of the inputs themselves: with the fast slope, every query
    row's running maximum over whole 32-token tiles rises by more than 2
    (log2 units) from each tile to the next up to the knee, so a kernel whose
    reference has 2 of headroom must rescale on every such tile."""
    w = _decode_workload(0.1, seed=71)
    oc = oracle_cache(w)
    kh, _ = attention.sequence_kv(oc, w.page_table[0], 1024, 0)
    q = codec.as_f32(w.q, w.dtype).astype(np.float64)[0, 0]
    s = (kh @ q) * w.softmax_scale * LOG2E
    tile_max = np.maximum.accumulate(s.reshape(-1, 32).max(axis=1))
    assert np.all(np.diff(tile_max) > 2.0)


@pytest.mark.gpu
@pytest.mark.parametrize("slope", SLOPES, ids=["fast", "slow", "falling"])
def test_decode_ramps(slope):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = _decode_workload(slope, seed=71)
    cache, want = upload_cache(w), oracle_out(w)
    for cfg in [None, dict(split_pages=64), dict(variant=5, split_pages=64), dict(variant=4, waves_per_wg=8),
                dict(fused_combine=1, split_pages=64)]:
        c = None if cfg is None else q8.make_config(**cfg)
        got = run_attention(w, cache, cfg=c)
        err = normalized_err(w, got, want)
        print(f"[ramp] decode slope {slope} cfg {cfg}: {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= ATOL_SIGMA, (slope, cfg, err)


@pytest.mark.gpu
@pytest.mark.parametrize("slope", SLOPES, ids=["fast", "slow", "falling"])
def test_verify_ramps(slope):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = _verify_workload(slope, seed=73)
    cache, want = upload_cache(w), oracle_out(w)
    for cfg in [None, dict(split_pages=64), dict(variant=5, waves_per_wg=4, split_pages=64),
                dict(fused_combine=1, split_pages=64)]:
        c = None if cfg is None else q8.make_config(**cfg)
        got = run_attention(w, cache, cfg=c)
        err = normalized_err(w, got, want)
        print(f"[ramp] verify slope {slope} cfg {cfg}: {err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= ATOL_SIGMA, (slope, cfg, err)


@pytest.mark.gpu
@pytest.mark.parametrize("slope", SLOPES, ids=["fast", "slow", "falling"])
def test_cascade_ramps(slope):
    from tests.gpu_util import run_prefix, upload_cache
    w = _sessions_workload(slope, seed=75)
    got = run_prefix(w, upload_cache(w), 1024 // 16)
    err = normalized_err(w, got, oracle_out(w))
    print(f"[ramp] cascade slope {slope}: {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err <= ATOL_SIGMA, (slope, err)
