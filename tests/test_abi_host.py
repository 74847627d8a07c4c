"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function the public header declares, and its argument validation
rejects bad calls before any device work."""

import ctypes as C
import os
import re
import subprocess

import pytest

import decode_attention_quantized_kv_amd as q8

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "q8k4v.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q8.LIB_PATH):
        pytest.skip("library not built")
    return q8.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("kv_quant_append", "attn_decode_q8k4v", "attn_verify_q8k4v", "tune_select",
              "attn_decode_prefix_q8k4v", "q8k4v_prefix_workspace_bytes", "attn_prefill_q8k4v",
              "q8k4v_hbm_probe", "q8k4v_stream_probe"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", q8.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    for n in _declared_functions():
        assert hasattr(lib, n)


def test_version_string(lib):
    assert q8.version().startswith("q8k4v 1 gfx950")


def _desc(head_dim=128, page_size=16):
    return q8.CacheDesc(4, 2, head_dim, page_size, 1, 1, 1, 1)


def test_append_rejects_bad_arguments(lib):
    d = _desc(head_dim=96)
    rc = lib.kv_quant_append(C.byref(d), 1, 1, 1, 1, 1, 1, 1, 1, 1, None)
    assert rc == -1 and b"head_dim" in lib.q8k4v_last_error()
    d = _desc(page_size=32)
    assert lib.kv_quant_append(C.byref(d), 1, 1, 1, 1, 1, 1, 1, 1, 1, None) == -1
    d = _desc()
    assert lib.kv_quant_append(C.byref(d), 1, 1, 7, 1, 1, 1, 1, 1, 1, None) == -1     # dtype
    assert lib.kv_quant_append(C.byref(d), None, 1, 1, 1, 1, 1, 1, 1, 1, None) == -1  # NULL k
    assert lib.kv_quant_append(C.byref(d), 1, 1, 1, 1, 1, 1, 1, 1, 0, None) == 0      # nothing to do
    assert lib.kv_quant_append(None, 1, 1, 1, 1, 1, 1, 1, 1, 1, None) == -1


def test_attention_rejects_bad_arguments(lib):
    d = _desc()
    args = dict(q=1, qd=1, out=1, n=1, hq=8, lens=1, msl=64, pt=1, mp=4)

    def dec(**kw):
        a = {**args, **kw}
        return lib.attn_decode_q8k4v(C.byref(d), a["q"], a["qd"], a["out"], a["n"], a["hq"], a["lens"], a["msl"],
                                     a["pt"], a["mp"], 0.1, None, None, 0, None)
    assert dec(hq=7) == -1                      # not a multiple of the kv heads
    assert dec(hq=6) == -2                      # group 3 unsupported
    assert dec(hq=32) == -2                     # group 16 unsupported
    assert dec(qd=5) == -1
    assert dec(mp=2) == -1                      # page table too short for max_seq_len
    assert dec(n=0) == -1
    assert dec(q=None) == -1
    assert lib.attn_verify_q8k4v(C.byref(d), 1, 1, 1, 1, 8, 17, 1, 64, 1, 4, 0.1, None, None, 0, None) == -1
    # prefill chunks: 1 .. 1024 new tokens, held by max_seq_len
    assert lib.attn_prefill_q8k4v(C.byref(d), 1, 1, 1, 1, 8, 1025, 1, 2048, 1, 128, 0.1, None, None, 0, None) == -1
    assert lib.attn_prefill_q8k4v(C.byref(d), 1, 1, 1, 1, 8, 0, 1, 64, 1, 4, 0.1, None, None, 0, None) == -1
    assert lib.attn_prefill_q8k4v(C.byref(d), 1, 1, 1, 1, 8, 100, 1, 64, 1, 4, 0.1, None, None, 0, None) == -1
    assert q8.workspace_bytes(1, 32, 8, 128, 65536, 1024) > 0
    assert lib.attn_verify_q8k4v(C.byref(d), 1, 1, 1, 1, 8, 3, 1, 2, 1, 4, 0.1, None, None, 0, None) == -1
    # workspace too small (needs split partials at this length)
    d2 = q8.CacheDesc(4096, 8, 128, 16, 1, 1, 1, 1)
    rc = lib.attn_decode_q8k4v(C.byref(d2), 1, 1, 1, 1, 32, 1, 65536, 1, 4096, 0.1, None, None, 0, None)
    assert rc == -3 and b"workspace" in lib.q8k4v_last_error()


WS_HEADER = 65536      # Q8K4V_WS_HEADER_BYTES


def test_workspace_size_follows_the_plan(lib):
    small = q8.workspace_bytes(1, 32, 8, 128, 64)
    big = q8.workspace_bytes(1, 32, 8, 128, 65536)
    assert big > 0 and big >= small
    cfg = q8.make_config(split_pages=32, variant=5)
    assert q8.workspace_bytes(1, 32, 8, 128, 512, 0, cfg) == 0       # one split: direct write, no workspace
    # variant 4 keeps at most 64 pages per wave: 4096 pages need splits
    assert q8.workspace_bytes(1, 32, 8, 128, 65536, 0, q8.make_config(split_pages=4096, variant=4)) > 0
    assert q8.workspace_bytes(1, 32, 8, 128, 65536, 0, q8.make_config(waves_per_wg=3)) == 0  # invalid config
    for v in (1, 2, 3, 6):                                             # only 0 (automatic), 4 and 5
        assert q8.workspace_bytes(1, 32, 8, 128, 4096, 0, q8.make_config(variant=v)) == 0
    assert q8.workspace_bytes(1, 4, 4, 128, 4096, 0, q8.make_config(tile_pages=4)) == 0


def test_sequences_that_fit_in_flight_are_not_split(lib):
    """The automatic plan does not split a sequence whose pages all fit in
    one workgroup's rings at once (waves x 2-page tiles x stages: 16 pages,
    256 tokens, at the decode defaults of 4 waves and 2 stages): no split
    records, so no workspace; one page more and it splits."""
    for hq, hkv, d in ((2, 1, 64), (32, 8, 128)):
        assert q8.workspace_bytes(1, hq, hkv, d, 256) == 0
        assert q8.workspace_bytes(4, hq, hkv, d, 256) == 0
        assert q8.workspace_bytes(1, hq, hkv, d, 257) > 0
    # 8 waves or 3 stages hold more pages in flight
    assert q8.workspace_bytes(1, 32, 8, 128, 512, 0, q8.make_config(waves_per_wg=8)) == 0
    assert q8.workspace_bytes(1, 32, 8, 128, 384, 0, q8.make_config(stages=3)) == 0
    assert q8.workspace_bytes(1, 32, 8, 128, 400, 0, q8.make_config(stages=3)) > 0
    # an explicit split length still splits
    assert q8.workspace_bytes(1, 32, 8, 128, 256, 0, q8.make_config(split_pages=8)) > 0


def test_workspace_header_is_shared_by_every_plan(lib):
    """Every plan that writes split records puts them behind one fixed
    header, and the in-launch merge keeps its counters inside that header:
    the fused and the separate merge need the same bytes, and no plan's
    records (decode, verify, prefill, cascade, at any length) can reach the
    counters of another.  (With the counters behind each plan's own records,
    a verify launch's records at 64K covered the 4K decode's counters.)"""
    shapes = [(1, 32, 8, 128, 4096, 0), (1, 32, 8, 128, 65536, 0), (1, 32, 8, 128, 65544, 8),
              (1, 32, 8, 128, 4104, 8), (1, 32, 8, 128, 65536 + 512, 512), (16, 32, 4, 128, 65536, 0)]
    for sh in shapes:
        plain = q8.workspace_bytes(*sh, q8.make_config(fused_combine=0))
        fused = q8.workspace_bytes(*sh, q8.make_config(fused_combine=1))
        assert plain == fused and plain > WS_HEADER, (sh, plain, fused)
        assert (plain - WS_HEADER) % 256 == 0
        # records: n_seqs x H x splits x rows x (D + 4) floats behind the header
        n, hq, h, d, _, nd = sh
        rows = (hq // h) * max(1, nd)
        assert (plain - WS_HEADER) >= n * h * 8 * rows * (d + 4) * 4
    pre = q8.prefix_workspace_bytes(16, 32, 4, 128, 65536, 2048)
    assert pre > WS_HEADER


def test_affine_cache_validation(lib):
    """An affine cache needs its zero-point pools; an unknown codec and an
    unknown kernel variant are refused (all before a launch)."""
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1, q8.CODEC_AFFINE, None, None)
    args = (1, 1, 1, 1, 32, 1, 64, 1, 4, 0.1)
    assert lib.attn_decode_q8k4v(C.byref(d), *args, None, None, 0, None) == -1
    assert b"k_zeros" in lib.q8k4v_last_error()
    assert lib.kv_quant_append(C.byref(d), 1, 1, 1, 1, 1, 1, 4, 1, 1, None) == -1
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1, 7, 1, 1)
    assert lib.attn_decode_q8k4v(C.byref(d), *args, None, None, 0, None) == -1
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1, q8.CODEC_AFFINE, 1, 1)
    for v in (1, 2, 3, 6):
        cfg = q8.make_config(variant=v)
        assert lib.attn_decode_q8k4v(C.byref(d), *args, C.byref(cfg), None, 0, None) == -1, v
        assert b"variant" in lib.q8k4v_last_error()


def test_prefix_cascade_validation_and_workspace(lib):
    """The shared-prefix entry point validates its page count on the host
    (before any launch) and sizes its workspace as prefix + suffix partials."""
    d = q8.CacheDesc(8192, 4, 128, 16, 1, 1, 1, 1)

    def casc(n_pref, msl=65536, mp=4096, n=16, hq=32, ws=None, wsb=0):
        return lib.attn_decode_prefix_q8k4v(C.byref(d), 1, 1, 1, n, hq, 1, msl, 1, mp, n_pref, 0.1, None, ws, wsb,
                                            None)
    assert casc(-1) == -1
    assert casc(4097) == -1                     # more pages than the page table holds
    assert casc(100, msl=1000) == -1            # prefix longer than max_seq_len
    assert casc(2048, hq=30) == -1              # bad head counts are still caught
    assert casc(2048, n=1024) == -2             # 1024 sessions x 8 rows: prefix block too large
    rc = casc(2048)                             # workspace missing
    assert rc == -3 and b"workspace" in lib.q8k4v_last_error()
    full = q8.workspace_bytes(16, 32, 4, 128, 65536)
    pre = q8.prefix_workspace_bytes(16, 32, 4, 128, 65536, 2048)
    assert pre > 0
    assert q8.prefix_workspace_bytes(16, 32, 4, 128, 65536, 0) == full
    assert q8.prefix_workspace_bytes(16, 32, 4, 128, 1000, 100) == 0
    # the prefix partials alone: 4 kv heads x splits x 128 rows x 132 floats
    assert pre >= 4 * 128 * 132 * 4
    # one session, whole context shared: still a valid cascade
    assert q8.prefix_workspace_bytes(1, 8, 8, 64, 4096, 256) > 0


def test_tuner_rejects_bad_requests(lib):
    """tune_select validates the request before touching the device."""
    def tune(**kw):
        r = q8.TuneRequest()
        base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=8, ctx_small=4096, ctx_large=65536,
                    budget_ms=1000)
        for k, v in {**base, **kw}.items():
            setattr(r, k, v)
        table = (q8.Config * 2)()
        return lib.tune_select(C.byref(r), table, None, 0)
    assert tune(num_q_heads=30) == -1           # not a multiple of the kv heads
    assert tune(num_q_heads=24) == -2           # group 3
    assert tune(head_dim=96) == -1
    assert tune(n_draft=0) == -1 and tune(n_draft=17) == -1
    assert tune(ctx_small=0) == -1
    assert tune(ctx_small=8192, ctx_large=4096) == -1
    assert lib.tune_select(None, None, None, 0) == -1
    # a reference term with a cache but an inconsistent length / table
    r = q8.TuneRequest()
    for k, v in dict(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=8, ctx_small=4096,
                     ctx_large=65536, budget_ms=1000).items():
        setattr(r, k, v)
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1)
    r.ref[2].cache = C.pointer(d)
    r.ref[2].q, r.ref[2].page_table, r.ref[2].out = 1, 1, 1
    r.ref[2].len, r.ref[2].max_pages = 4, 64          # verify term shorter than its 8 drafts
    table = (q8.Config * 2)()
    assert lib.tune_select(C.byref(r), table, None, 0) == -1 and b"term 2" in lib.q8k4v_last_error()
    r.ref[2].len, r.ref[2].max_pages = 4104, 64       # 64 pages cannot hold 4104 tokens
    assert lib.tune_select(C.byref(r), table, None, 0) == -1


def test_tuner_rejects_bad_session_requests(lib):
    """The multi-session unit: a session count of 2..64, and its reference
    terms only with it and with their lengths, sessions and prefix."""
    def req(**kw):
        r = q8.TuneRequest()
        for k, v in {**dict(num_q_heads=32, num_kv_heads=8, head_dim=128, n_draft=8, ctx_small=4096,
                            ctx_large=65536, budget_ms=1000), **kw}.items():
            setattr(r, k, v)
        return r
    table = (q8.Config * 3)()
    for ns in (1, -2, 65):
        assert lib.tune_select(C.byref(req(n_sessions=ns)), table, None, 0) == -1
        assert b"n_sessions" in lib.q8k4v_last_error()
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1)
    def with_ref(ns, **kw):
        r = req(n_sessions=ns)
        t = r.ref[4]
        t.cache = C.pointer(d)
        t.q, t.page_table, t.out, t.seq_lens = 1, 1, 1, 1
        t.len, t.max_pages, t.n_seqs, t.n_prefix_pages = 600, 64, 4, 16
        for k, v in kw.items():
            setattr(t, k, v)
        return lib.tune_select(C.byref(r), table, None, 0)
    assert with_ref(0) == -1 and b"needs n_sessions" in lib.q8k4v_last_error()
    assert with_ref(4, seq_lens=None) == -1 and b"term 4" in lib.q8k4v_last_error()
    assert with_ref(4, n_seqs=0) == -1
    assert with_ref(4, n_prefix_pages=0) == -1
    assert with_ref(4, n_prefix_pages=65) == -1     # more shared pages than the table holds
    assert with_ref(4, len=200) == -1               # shorter than the shared prefix
    assert with_ref(4, n_seqs=1100) == -1           # 1100 sessions x 4 rows: prefix block too large


def test_binding_rejects_host_tensors():
    """The binding hands raw device pointers to the library: host tensors are
    refused before any call (no CPU path)."""
    import torch
    import decode_attention_quantized_kv_amd as q8
    with pytest.raises(ValueError):
        q8._ptr(torch.zeros(4), "q")
    with pytest.raises(ValueError):
        q8._ptr(torch.zeros(4, dtype=torch.int32), "seq_lens", i32=True)
    assert q8._ptr(None).value is None


def test_long_context_splits_are_even(lib):
    """Beyond the 64-pages-per-wave cap, a one-chunk decode takes a whole
    number of workgroups per CU and a multiple of 8 splits (the workspace
    holds one (m, l, o[D]) record per split, kv head and row); prefill blocks
    keep the capped split, and no plan pads its split count."""
    import decode_attention_quantized_kv_amd as q8
    rec = 4 * (128 + 4)

    def splits(ctx, n_new=0):
        rows = 4 * max(1, n_new)
        return (q8.workspace_bytes(1, 32, 8, 128, ctx, n_new) - WS_HEADER) / (8 * rows * rec)

    assert splits(65536) == 32 and splits(131072) == 32       # under the cap: one workgroup per CU
    for ctx in (163840, 200000, 262144):
        s = splits(ctx)
        assert 62 <= s <= 64, (ctx, s)                       # about two per CU (whole tiles per split)
    assert splits(65536 + 512, 512) == 9                     # 9 capped splits (no padding)


def test_probes_reject_bad_arguments(lib):
    """The streaming probes validate before any launch."""
    d = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1)
    assert lib.q8k4v_hbm_probe(C.byref(d), 1, 1, 1024, 1, 64, 4, 5, 1, None) == -1       # stages
    assert lib.q8k4v_hbm_probe(C.byref(d), 1, 1, 1024, 1, 64, 2, 2, 1, None) == -1       # waves
    assert lib.q8k4v_hbm_probe(C.byref(d), 1, 1, 1024, 1, 64, 4, 3, 8, None) == -1       # 8 heads need 8 waves
    assert lib.q8k4v_hbm_probe(C.byref(d), 1, 1, 1024, 1, 64, 4, 3, 3, None) == -1       # heads per workgroup
    da = q8.CacheDesc(64, 8, 128, 16, 1, 1, 1, 1, q8.CODEC_AFFINE, 1, 1)
    assert lib.q8k4v_hbm_probe(C.byref(da), 1, 1, 1024, 1, 64, 4, 3, 1, None) == -1      # symmetric only
    assert lib.q8k4v_stream_probe(None, 4096, 4, 3, None) == -1
    assert lib.q8k4v_stream_probe(16, 1000, 4, 3, None) == -1                         # too short
    assert lib.q8k4v_stream_probe(16, 4100, 4, 3, None) == -1                         # not a multiple of 16
    assert lib.q8k4v_stream_probe(16, 4096, 4, 5, None) == -1
