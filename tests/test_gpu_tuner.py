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


def test_tuner_search_order_follows_virtual_completion_time():
    """After the defaults, each measured candidate came from the unit with the
    earliest virtual completion time (effort + price) / (share x opportunity)
    at that moment, and both units were searched."""
    dcfg, vcfg, rep, _ = _tune(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=8, ctx_small=1024,
                               ctx_large=8192, budget_ms=6000, seed=7)
    assert rep["status"] == "searched"
    picked = sorted((c["seq"], u, c) for u, cands in enumerate(rep["candidates"]) for c in cands
                    if c["stage"] != "default" and c["seq"] >= 0)
    assert {u for _, u, _ in picked} == {0, 1}
    assert [s for s, _, _ in picked] == list(range(2, 2 + len(picked)))   # the defaults are 0 and 1
    for _, u, c in picked:
        mine, other = c["vt"][u], c["vt"][1 - u]
        assert mine is not None and mine > 0
        assert other is None or mine <= other


def test_tuner_records_reuse_and_identity_change(tmp_path):
    path = str(tmp_path / "tune.rec")
    kw = dict(num_q_heads=16, num_kv_heads=4, head_dim=128, n_draft=4, ctx_small=512, ctx_large=4096,
              budget_ms=4000, seed=6, record_path=path)
    d1, v1, rep1, _ = _tune(**kw)
    assert rep1["status"] == "searched" and rep1["record"] == "stored"
    ident = rep1["identity_hash"]
    assert "arch=gfx950" in rep1["identity"] and "library=q8k4v" in rep1["identity"]
    lines = open(path).read().splitlines()
    assert len(lines) == 2 and all(l.split()[:3] == ["q8k4v-tune-record", "1", ident] for l in lines)
    # the same identity and shape: the stored choice, nothing measured
    d2, v2, rep2, wall = _tune(**kw)
    assert rep2["status"] == "stored" and rep2["record"] == "loaded"
    assert rep2["elapsed_ms"] < 500 and all(len(c) == 0 for c in rep2["candidates"])
    assert d2.as_dict() == d1.as_dict() and v2.as_dict() == v1.as_dict()
    # another shape keeps its own records beside the first ones
    _tune(**{**kw, "n_draft": 2})
    assert len(open(path).read().splitlines()) == 4
    # another identity (a new driver, toolchain or library build) searches again
    # and keeps the other identity's records; unreadable lines are dropped
    text = open(path).read()
    with open(path, "w") as f:
        f.write(text.replace(ident, "0123456789abcdef") + "not a record\n")
    d3, v3, rep3, _ = _tune(**kw)
    assert rep3["status"] == "searched" and rep3["record"] == "stored"
    hashes = [l.split()[2] for l in open(path).read().splitlines()]
    assert hashes.count("0123456789abcdef") == 4 and hashes.count(ident) == 2 and len(hashes) == 6
