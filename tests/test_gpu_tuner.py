"""GPU tests of tune_select, the on-device launch-configuration tuner (the
first-load tuner of blog.123qwe.co.kr/?p=3927, section 3, admission rule of
section 4): the wall-clock budget holds, timing rotates past the last-level
cache, every admitted configuration reproduces the oracle, a tiny budget or
failing references leave the defaults unqualified, and installed winners are
used by calls without a config."""

import json
import time

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


def _tune(**kw):
    import decode_attention_quantized_kv_amd as q8
    t0 = time.perf_counter()
    dcfg, vcfg, rep = q8.tune_select(**kw)
    wall = time.perf_counter() - t0
    print("[tuner]", json.dumps({k: v for k, v in rep.items() if k != "candidates"}), flush=True)
    return dcfg, vcfg, rep, wall


def _parity(cfg, hq, hkv, D, n_draft):
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_attention, upload_cache
    w = workloads.build("tp", seed=21 + n_draft, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype="bf16",
                        seq_lens=[900, n_draft + 37], n_draft=n_draft if n_draft > 1 else 0, outliers=True)
    cache = upload_cache(w)
    c = None if cfg is None else q8.make_config(**{k: v for k, v in cfg.as_dict().items() if k != "qualified"})
    err = normalized_err(w, run_attention(w, cache, cfg=c), oracle_out(w))
    assert err <= ATOL_SIGMA, err


def test_tuner_budget_rotation_and_admitted_parity():
    budget = 8000
    dcfg, vcfg, rep, wall = _tune(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=8, ctx_small=1024,
                                  ctx_large=16384, budget_ms=budget, seed=5)
    assert rep["status"] == "searched"
    assert rep["elapsed_ms"] <= budget + 1500, rep["elapsed_ms"]
    assert wall * 1e3 <= budget + 3000, wall
    assert rep["rotation"]["llc_multiple"] >= 4.0
    assert len(rep["units"]) == 2 and len(rep["candidates"]) == 2
    for unit, cfg, cands in zip(rep["units"], (dcfg, vcfg), rep["candidates"]):
        assert unit["searched"] == len(cands) >= 2
        assert cands[0]["stage"] == "default" and cands[0]["verdict"] == "admitted"
        assert unit["qualified"] and cfg.qualified == 1
        assert unit["chosen_cost"] <= 2.0 + 1e-9
        for c in cands:
            if c["verdict"] == "admitted":
                assert c["us"][0] > 0 and c["us"][1] > 0
                assert max(c["dev"]) <= rep["alpha"] * max(unit["noise"])
        chosen = unit["chosen"]
        assert {k: getattr(cfg, k) for k in chosen} == chosen
        # the noise floor is real: moving every code by one step moves the output
        assert min(unit["noise"]) > 0
    _parity(dcfg, 32, 8, 128, 1)
    _parity(vcfg, 32, 8, 128, 8)


def test_tuner_tiny_budget_leaves_defaults_unqualified():
    dcfg, vcfg, rep, wall = _tune(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=4, ctx_small=256,
                                  ctx_large=4096, budget_ms=0, seed=1)
    assert dcfg.qualified == 0 and vcfg.qualified == 0
    assert not rep["installed"]
    for unit in rep["units"]:
        assert not unit["qualified"]
        assert unit["admitted"] <= 1       # at most the default, never a measured winner


def test_tuner_memory_admission_refuses():
    import decode_attention_quantized_kv_amd as q8
    with pytest.raises(q8.Q8K4VError) as e:
        q8.tune_select(num_q_heads=8, num_kv_heads=2, head_dim=128, n_draft=2, ctx_small=1024, ctx_large=65536,
                       budget_ms=5000, mem_cap_bytes=1 << 20)
    assert e.value.code == -5


def _reference(hq, hkv, D, W, L, seed):
    """Caller references: the oracle's verify output on a small cache and the
    decode output of the last draft's query at the full length."""
    from tests.gpu_util import to_dev, upload_cache
    w = workloads.build("tref", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype="bf16",
                        seq_lens=[L], n_draft=W, outliers=False)
    cache = upload_cache(w)
    want = oracle_out(w)                     # [1][W][Hq][D]
    return w, {
        "cache": cache,
        "q": to_dev(np.ascontiguousarray(w.q[0, W - 1]), "bf16"),
        "q_verify": to_dev(np.ascontiguousarray(w.q[0]), "bf16"),
        "page_table": to_dev(np.ascontiguousarray(w.page_table[0])),
        "length": L,
        "out": want[0, W - 1].astype(np.float32),
        "out_verify": want[0].astype(np.float32),
        "tol": ATOL_SIGMA,
    }


def test_tuner_reference_gate_and_install():
    hq, hkv, D, W = 16, 4, 64, 3
    w, ref = _reference(hq, hkv, D, W, 1500, seed=77)
    dcfg, vcfg, rep, _ = _tune(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=W, ctx_small=512,
                               ctx_large=8192, budget_ms=6000, seed=3, install=True, ref=ref)
    assert rep["installed"]
    for unit, cands in zip(rep["units"], rep["candidates"]):
        assert unit["qualified"]
        for c in cands:
            if c["verdict"] == "admitted":
                assert c["ref_dev"] <= ATOL_SIGMA
    # installed winners serve calls without a config, still at parity
    _parity(None, hq, hkv, D, 1)
    _parity(None, hq, hkv, D, W)


def test_tuner_wrong_references_admit_nothing():
    hq, hkv, D, W = 8, 8, 64, 2
    w, ref = _reference(hq, hkv, D, W, 700, seed=78)
    ref["out"] = ref["out"] + 0.5            # references planted wrong on the host
    ref["out_verify"] = ref["out_verify"] + 0.5
    dcfg, vcfg, rep, _ = _tune(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=W, ctx_small=512,
                               ctx_large=4096, budget_ms=4000, seed=4, install=True, ref=ref)
    assert dcfg.qualified == 0 and vcfg.qualified == 0
    for unit, cands in zip(rep["units"], rep["candidates"]):
        assert not unit["qualified"] and unit["admitted"] == 0
        assert cands[0]["verdict"] == "rejected"
