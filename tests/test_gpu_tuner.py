"""GPU tests of tune_select, the on-device launch-configuration tuner (the
first-load tuner of blog.123qwe.co.kr/?p=3927, section 3, admission rule of
section 4): the wall-clock budget holds, timing rotates past the last-level
cache, every admitted configuration reproduces the oracle, a tiny budget or
failing references leave the defaults unqualified, and installed winners are
used by calls without a config; with n_sessions the multi-session unit (the
shared-prefix entry point's suffix pass) is searched and gated the same way."""

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
    dcfg, vcfg, _, rep = q8.tune_select(**kw)
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
        assert unit["invalid"] == 0, unit["invalid_why"]   # no candidate the library refuses
        for c in cands:
            if c["verdict"] == "admitted":
                assert c["us"][0] > 0 and c["us"][1] > 0
                assert max(c["dev"]) <= rep["alpha"] * max(unit["noise"])
            if c["verdict"] == "rejected":
                assert c["gate"] == "alpha" and c["why"]
            # a deviation is null only when it was not measured (deadline or
            # an earlier rejection), never reported as 0
            if c["verdict"] == "admitted":
                assert all(d is not None for d in c["dev"])
        # in-launch-merge candidates write their outputs on both shapes (one
        # workspace serves every candidate of both units)
        fused = [c for c in cands if c["cfg"]["fused_combine"] == 1 and c["verdict"] != "unknown"]
        assert fused and all(c["dev"][0] is not None and c["verdict"] == "admitted" for c in fused), \
            [(c["cfg"], c["verdict"], c.get("why")) for c in fused if c["verdict"] != "admitted"]
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


def _references(hq, hkv, D, W, L_small, L_large, seed):
    """Oracle references for the tuner's four terms on caller inputs: decode
    and verify at a small and a large context (two sequences with W drafts
    appended; decode attends the context before the drafts)."""
    from oracle import attention
    from tests.gpu_util import to_dev, upload_cache
    from tests.util import oracle_cache, sigma_q_heads
    refs = {}
    for size, L in (("small", L_small), ("large", L_large)):
        w = workloads.build("tref_" + size, seed=seed + L, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                            dtype="bf16", seq_lens=[L + W], n_draft=W, outliers=True)
        cache, oc = upload_cache(w), oracle_cache(w)
        ver = oracle_out(w, oc)                                        # [1][W][Hq][D]
        qd = np.ascontiguousarray(w.q[:, 0])                           # [1][Hq][D]
        dec = attention.decode(oc, qd, w.dtype, w.page_table, np.array([L], np.int32), w.softmax_scale)
        pt = to_dev(np.ascontiguousarray(w.page_table[0]))
        sig = sigma_q_heads(w)
        refs["decode_" + size] = {"cache": cache, "q": to_dev(qd[0], "bf16"), "page_table": pt, "length": L,
                                  "out": dec[0].astype(np.float32), "sigma": sig}
        refs["verify_" + size] = {"cache": cache, "q": to_dev(np.ascontiguousarray(w.q[0]), "bf16"),
                                  "page_table": pt, "length": L + W, "out": ver[0].astype(np.float32), "sigma": sig}
    return refs


def test_tuner_reference_gate_and_install():
    hq, hkv, D, W = 16, 4, 64, 3
    refs = _references(hq, hkv, D, W, 512, 3000, seed=77)
    dcfg, vcfg, rep, _ = _tune(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=W, ctx_small=512,
                               ctx_large=8192, budget_ms=6000, seed=3, install=True, refs=refs,
                               ref_tol=ATOL_SIGMA)
    assert rep["installed"]
    for unit, cands in zip(rep["units"], rep["candidates"]):
        assert unit["qualified"] and unit["oracle_gate"] == [True, True]
        for c in cands:
            if c["verdict"] == "admitted":
                assert max(c["ref_dev"]) <= ATOL_SIGMA
    # installed winners serve calls without a config, still at parity
    _parity(None, hq, hkv, D, 1)
    _parity(None, hq, hkv, D, W)


def test_tuner_wrong_references_admit_nothing():
    hq, hkv, D, W = 8, 8, 64, 2
    refs = _references(hq, hkv, D, W, 300, 700, seed=78)
    for r in refs.values():
        r["out"] = r["out"] + 0.5            # references planted wrong on the host
    dcfg, vcfg, rep, _ = _tune(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=W, ctx_small=512,
                               ctx_large=4096, budget_ms=4000, seed=4, install=True, refs=refs,
                               ref_tol=ATOL_SIGMA)
    assert dcfg.qualified == 0 and vcfg.qualified == 0
    for unit, cands in zip(rep["units"], rep["candidates"]):
        assert not unit["qualified"] and unit["admitted"] == 0
        assert cands[0]["verdict"] == "rejected" and cands[0]["gate"] == "oracle"


def test_tuner_one_wrong_term_rejects_the_unit():
    """Every term is gated: a reference wrong on the large verify term alone
    leaves the verify unit unqualified and the decode unit qualified."""
    hq, hkv, D, W = 8, 2, 128, 4
    refs = _references(hq, hkv, D, W, 300, 1200, seed=79)
    refs["verify_large"]["out"] = refs["verify_large"]["out"] * 1.01 + 0.05
    dcfg, vcfg, rep, _ = _tune(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=W, ctx_small=512,
                               ctx_large=4096, budget_ms=4000, seed=5, refs=refs,
                               ref_tol=ATOL_SIGMA)
    assert dcfg.qualified == 1 and vcfg.qualified == 0
    ver = rep["candidates"][1][0]
    assert ver["verdict"] == "rejected" and ver["gate"] == "oracle" and "term 3" in ver["why"]


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
    assert len(lines) == 2 and all(l.split()[:3] == ["q8k4v-tune-record", "2", ident] for l in lines)
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


def _session_references(hq, hkv, D, ns, seed):
    """Oracle references for the multi-session terms: ns ragged sessions over
    a 256-token (small) and a 2048-token (large) shared prefix."""
    from tests.gpu_util import to_dev, upload_cache
    from tests.util import sigma_q_heads
    rng = np.random.default_rng(seed)
    refs = {}
    for size, pre, suf in (("small", 256, 300), ("large", 2048, 1500)):
        w = workloads.build("tref_ms_" + size, seed=seed + pre, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                            dtype="bf16", seq_lens=pre + rng.integers(0, suf, size=ns), shared_prefix=pre,
                            outliers=True)
        refs["multi_session_" + size] = {
            "cache": upload_cache(w), "q": to_dev(w.q, "bf16"), "page_table": to_dev(w.page_table),
            "length": int(max(w.seq_lens)), "seq_lens": to_dev(w.seq_lens), "n_prefix_pages": pre // 16,
            "out": oracle_out(w).astype(np.float32), "sigma": sigma_q_heads(w)}
    return refs


def test_tuner_multi_session_unit():
    """n_sessions adds a third unit: it is searched in the same virtual-time
    order, never with the in-launch merge, every admitted candidate matches
    the oracle on both multi-session terms, and the installed winner serves
    the shared-prefix entry point without a config, at parity."""
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import run_prefix, upload_cache
    hq, hkv, D, NS = 16, 4, 128, 4
    refs = _session_references(hq, hkv, D, NS, seed=80)
    t0 = time.perf_counter()
    dcfg, vcfg, mcfg, rep = q8.tune_select(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, n_draft=4,
                                           ctx_small=1024, ctx_large=8192, budget_ms=9000, seed=8, install=True,
                                           refs=refs, ref_tol=ATOL_SIGMA, n_sessions=NS)
    wall = time.perf_counter() - t0
    print("[tuner]", json.dumps({k: v for k, v in rep.items() if k != "candidates"}), flush=True)
    assert rep["status"] == "searched" and wall * 1e3 <= 9000 + 3000
    assert len(rep["units"]) == 3 and len(rep["candidates"]) == 3
    ms, cands = rep["units"][2], rep["candidates"][2]
    assert ms["unit"] == "multi_session" and ms["sessions"] == NS and ms["rows_per_kv_head"] == hq // hkv
    assert ms["oracle_gate"] == [True, True] and rep["units"][0]["oracle_gate"] == [False, False]
    assert ms["invalid"] == 0, ms["invalid_why"]
    assert cands[0]["stage"] == "default" and cands[0]["verdict"] == "admitted" and len(cands) >= 2
    assert ms["qualified"] and mcfg.qualified == 1
    assert {k: getattr(mcfg, k) for k in ms["chosen"]} == ms["chosen"]
    for c in cands:
        assert c["cfg"]["fused_combine"] == 0
        if c["verdict"] == "admitted":
            assert max(c["ref_dev"]) <= ATOL_SIGMA
            assert max(c["dev"]) <= rep["alpha"] * max(ms["noise"])
    # the order over three units: each pick had the least virtual time
    picked = [(u, c) for u, cs in enumerate(rep["candidates"]) for c in cs if c["stage"] != "default" and c["seq"] >= 0]
    assert 2 in {u for u, _ in picked}
    for u, c in picked:
        assert len(c["vt"]) == 3 and c["vt"][u] is not None
        assert all(v is None or c["vt"][u] <= v for v in c["vt"])
    # the installed winner serves calls without a config
    w = workloads.build("ms_after_tune", seed=81, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, dtype="bf16",
                        seq_lens=[700, 513, 1200, 512, 999], shared_prefix=512, outliers=True)
    err = normalized_err(w, run_prefix(w, upload_cache(w), 32), oracle_out(w))
    assert err <= ATOL_SIGMA, err
