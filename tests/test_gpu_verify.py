"""GPU parity of attn_verify_q8k4v against the fp64 oracle: draft widths
and group sizes on both kernels (the replicated-row kernel for 1, 2, 4, 8 or
16 rows per kv head, the row-block kernel otherwise), the causal rule among drafts (verify row j equals a decode at length L-W+j+1),
ragged batches, and the full 64K verify workload."""

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu


def _check(w, got, want, label):
    err = normalized_err(w, got, want)
    print(f"[verify] {label}: max |err|/sigma = {err:.3e}", flush=True)
    assert err <= ATOL_SIGMA, (label, err)
    return err


@pytest.mark.parametrize("W,hq,hkv,D", [(2, 8, 4, 128), (2, 16, 8, 128), (4, 8, 8, 128), (1, 32, 8, 128),
                                         (8, 32, 8, 128), (4, 32, 8, 128), (3, 32, 8, 128), (16, 32, 8, 128),
                                         (8, 32, 8, 64), (5, 8, 8, 64), (8, 32, 4, 128), (16, 64, 8, 128)])
def test_draft_widths_and_groups(W, hq, hkv, D):
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("ver", seed=W * 100 + hq + D, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype="bf16",
                        seq_lens=[W, W + 13, 700, 1037], n_draft=W, outliers=True)
    cache = upload_cache(w)
    _check(w, run_attention(w, cache), oracle_out(w), f"W={W} hq={hq} hkv={hkv} D={D}")


def test_verify_rows_equal_decodes_on_gpu():
    """Row j of a verify equals a decode of the same query at length L-W+j+1
    (both on the GPU, within the tolerance of each against the oracle)."""
    from tests.gpu_util import run_attention, upload_cache
    W = 8
    w = workloads.build("cv", seed=7, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[333, 1500], n_draft=W, outliers=True)
    cache = upload_cache(w)
    ver = run_attention(w, cache)
    for j in range(W):
        lens = (w.seq_lens - W + j + 1).astype(np.int32)
        dec = run_attention(w, cache, q=np.ascontiguousarray(w.q[:, j]), seq_lens=lens)
        err = normalized_err(w, ver[:, j], dec)
        assert err <= ATOL_SIGMA, (j, err)


@pytest.mark.parametrize("cfg", [dict(waves_per_wg=2), dict(waves_per_wg=4), dict(fused_combine=1),
                                 dict(split_pages=2), dict(wgs_per_cu=6), dict(variant=5, stages=3), dict(variant=5, waves_per_wg=8, stages=3),
                                 dict(variant=5, waves_per_wg=2, stages=2, fused_combine=1),
                                 dict(variant=5, waves_per_wg=4, stages=3, fused_combine=1), dict(wgs_per_cu=2)],
                         ids=str)
def test_verify_launch_configurations(cfg):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("vcfg", seed=11, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        seq_lens=[1200, 77], n_draft=8, outliers=True)
    cache = upload_cache(w)
    _check(w, run_attention(w, cache, cfg=q8.make_config(**cfg)), oracle_out(w), f"cfg {cfg}")


@pytest.mark.slow
def test_full_64k_verify():
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.verify_64k()
    cache = upload_cache(w)
    _check(w, run_attention(w, cache), oracle_out(w), "verify_65536_w8")
